// train.hip -- gfx950 kernels of the text encoder's backward pass and of the Adafactor update.
//
// What is computed: "UForm" page, "Precision by Design" (bf16 storage and matrix products with fp32
// accumulation; gradients accumulated in fp32 and cast to bf16 for the update; optionally every block's
// backward replays its forward from the block's fp32 input) and "Adafactor Optimizer" (factored second
// moment, clipped update, first moment with Adam's bias correction; bf16 master weights, fp32 norm gains).
//
// The products of the backward pass reuse the forward's GEMM kernel (activation gradients: dY W^T reads
// the canonical [in x out] weights, which are K-contiguous for that product). This file adds the weight
// gradients X^T Y (both operands token-major: read through the LDS transpose load), attention backward
// (with the rotary's transpose in its stores), and the row kernels (RMSNorm and SwiGLU backward, the pool
// and the byte embedding), the multi-tensor Adafactor and the repacking of derived weight copies.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "device.h"
#include "train.h"

namespace ube {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));


__device__ __forceinline__ s16x4 tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
    const s16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

// Tiles of 128-byte rows that are read both along their rows (16-byte reads) and down them (transpose
// reads): the 16-byte chunks of row r are XOR-swizzled by m ^ 4 (m % 2), m = (r / 2) % 8. That is a
// permutation of 0..7, so 16 consecutive rows read at one logical chunk hit 16 distinct bank groups, and
// the four rows 4j .. 4j + 3 that one transpose read covers (8 bytes from each of four chunks per row)
// land in four distinct 64-byte bank ranges: no bank conflicts either way.
__device__ __forceinline__ int swzb(int row, int ch) {
    const int m = (row >> 1) & 7;
    return ch ^ m ^ ((m & 1) << 2);
}

// MFMA A operand whose k runs down the rows of an LDS tile [rows][64 bf16] (128-byte rows, 16-byte chunks
// swizzled by swzb): lane l receives column c0 + l % 32 at the 8 k slots of half hh = l / 32, slot q being
// row kb + 4 hh + (q % 4) + 8 (q / 4) -- the order in which a 32x32 MFMA result holds its rows in
// registers 8s .. 8s + 7 (kb = 16 s), so such an accumulator, packed to bf16, is the matching B operand.
// ds_read_b64_tr_b16: lane i = 4a + b of a 16-lane group receives element b of the 8 bytes read by lanes
// 4e + a of the group, as its element e.
__device__ __forceinline__ bf16x8 tr_rows_frag(const uint8_t *tile, int kb, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15, hh = g >> 1;
    const int col = c0 + 16 * (g & 1) + 4 * (i & 3);
    const int chunk = col >> 3, half = (col >> 2) & 1;
    const int r0 = kb + 4 * hh + (i >> 2), r1 = r0 + 8;
    const uint8_t *p0 = tile + r0 * 128 + (swzb(r0, chunk) << 4) + (half << 3);
    const uint8_t *p1 = tile + r1 * 128 + (swzb(r1, chunk) << 4) + (half << 3);
    return join(tr16(p0), tr16(p1));
}

// MFMA operand whose k runs down the rows of an LDS tile of PITCH-byte rows in plain k order (rows kb + 8 hh
// + 0..7), chunks XOR-swizzled by 4 ((r / 2) % 2) (128-byte rows) or 4 (r % 4) (256 bytes and more).
template <int PITCH>
__device__ __forceinline__ int kmajor_swz(int r) {
    return PITCH == 128 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

template <int PITCH>
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t *tile, int kb, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int col = c0 + 16 * (g & 1) + 4 * (i & 3);
    const int chunk = col >> 3, half = (col >> 2) & 1;
    const int r0 = kb + 8 * (g >> 1) + (i >> 2), r1 = r0 + 4;
    const uint8_t *p0 = tile + r0 * PITCH + ((chunk ^ kmajor_swz<PITCH>(r0)) << 4) + (half << 3);
    const uint8_t *p1 = tile + r1 * PITCH + ((chunk ^ kmajor_swz<PITCH>(r1)) << 4) + (half << 3);
    return join(tr16(p0), tr16(p1));
}

__device__ __forceinline__ bf16x8 pack8(const f32x16 &v, int s) {
    const u32x4 w = {pack2(v[8 * s], v[8 * s + 1]), pack2(v[8 * s + 2], v[8 * s + 3]), pack2(v[8 * s + 4], v[8 * s + 5]),
                     pack2(v[8 * s + 6], v[8 * s + 7])};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ u32x4 load16(const uint16_t *p) { return *(const u32x4 *)p; }

// ----------------------------------------------------------------------------------- attention backward
//
// Notation per head: s = q.k / 8 (natural units), P = softmax over the item's keys, rebuilt as
// 2^(log2(e) s - lse) from the forward's base-2 log denominators; dP = dO V^T; dS = P (dP - delta) with
// delta = rowsum(dO O); dQ = dS K / 8, dK = dS^T Q / 8, dV = P^T dO.
// Two kernels, 8 waves x 32 rows per workgroup (one 256-token tile of one item and head), 64-row tiles of
// the other side double-buffered in LDS by DMA (16-byte chunks swizzled by swzb; V^T by kmajor_swz):
//   dQ: S^T = K Q^T and dP^T = V dO^T (a lane holds one query and 16 keys), dQ^T += K^T dS^T;
//   dK, dV: S = Q K^T and dP = dO V^T (a lane holds one key and 16 queries), dV^T += dO^T P,
//           dK^T += Q^T dS.
// The second product of each pair reads its A operand through the transpose load in the row order of the
// accumulator, so the accumulators feed it as B operands without leaving registers.

constexpr float kScale2 = 0.18033688011112042f;  // log2(e) / 8

// The transpose of the rotary map on two adjacent pairs (g0, g1), (g2, g3) with cs = (cos, sin) of each:
// (g0, g1) -> (c g0 + s g1, -s g0 + c g1), the gradient with respect to the values before the rotation.
__device__ __forceinline__ void unrotate4(float (&g)[4], f32x4 cs) {
    const float a0 = cs.x * g[0] + cs.y * g[1], a1 = -cs.y * g[0] + cs.x * g[1];
    const float b0 = cs.z * g[2] + cs.w * g[3], b1 = -cs.w * g[2] + cs.z * g[3];
    g[0] = a0, g[1] = a1, g[2] = b0, g[3] = b1;
}

__global__ __launch_bounds__(512, 4) void k_attn_bwd_dq(AttnBwdArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[4 * 1024];  // stage: K tile 512 | V tile 512 chunks
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int head = logical / a.ntiles, ti = logical % a.ntiles;
    const int2 tile = a.tiles[ti];
    const int k0 = a.cu[tile.x], k1 = a.cu[tile.x + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int qbase = tile.y + wave * 32;
    const bool active = qbase < k1;
    const bool qvalid = qbase + l32 < k1;
    const int t = min(qbase + l32, k1 - 1);
    bf16x8 qf[4], dof[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qf[ks] = __builtin_bit_cast(bf16x8, load16(a.q + (size_t)t * a.ldqk + head * 64 + ks * 16 + hh * 8));
        dof[ks] = __builtin_bit_cast(bf16x8, load16(a.dout + (size_t)t * a.lddo + head * 64 + ks * 16 + hh * 8));
    }
    // delta = rowsum(dO * O) of this lane's query over the head's 64 features (lane half hh holds 32 of
    // them), written for the dK/dV kernel that runs next
    float dlt = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ov = load16(a.o + (size_t)t * a.ldo + head * 64 + ks * 16 + hh * 8);
        const u32x4 dv = __builtin_bit_cast(u32x4, dof[ks]);
        const uint32_t o4[4] = {ov.x, ov.y, ov.z, ov.w}, d4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dlt += bf16_to_f32(o4[q] & 0xffff) * bf16_to_f32(d4[q] & 0xffff) +
                   bf16_to_f32(o4[q] >> 16) * bf16_to_f32(d4[q] >> 16);
    }
    dlt += __shfl_xor(dlt, 32, 64);
    if (hh == 0 && qvalid) a.delta[(size_t)head * a.ldl + t] = dlt;
    const float lse2 = a.lse[(size_t)head * a.ldl + t];
    const int prow = tid >> 3, pc = swzb(prow, tid & 7), pv = (tid & 7) ^ kmajor_swz<128>(prow);
    // K tile: 64 key rows of the head's 64 features; V^T tile: the head's 64 feature rows of vt over the
    // tile's 64 keys (k-major for dP^T = V dO^T, read with the transpose load). Keys past the item read
    // other items' values or the zeroed band after the last token: finite, and weighted 0.
    auto issue = [&](int tt, int buf) {
        const int row = min(k0 + tt * 64 + prow, k1 - 1);
        u32x4 *dst = smem + buf * 1024;
        lds_dma16(a.k + (size_t)row * a.ldqk + head * 64 + pc * 8, dst + wave * 64);
        lds_dma16(a.vt + (size_t)(head * 64 + prow) * a.ldvt + k0 + tt * 64 + pv * 8, dst + 512 + wave * 64);
    };
    f32x16 dQ[2] = {f32x16{}, f32x16{}};
    const int ntile = (k1 - k0 + 63) >> 6;
    // key tiles in pairs over four buffers: one barrier per pair publishes both tiles and retires every
    // wave's reads of the previous pair, whose buffers then receive the next pair
    issue(0, 0);
    if (1 < ntile) issue(1, 1);
    for (int tp = 0; tp < ntile; tp += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        if (tp + 2 < ntile) issue(tp + 2, (tp + 2) & 3);
        if (tp + 3 < ntile) issue(tp + 3, (tp + 3) & 3);
        if (!active) continue;
        for (int tt = tp; tt < min(tp + 2, ntile); ++tt) {
        const u32x4 *sK = smem + (tt & 3) * 1024, *sVt = sK + 512;
        const int kt = k0 + tt * 64;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x16 S = f32x16{}, dP = f32x16{};
            const int row = kk * 32 + l32;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int ch = swzb(row, ks * 2 + hh);
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sK[row * 8 + ch]), qf[ks], S, 0, 0, 0);
                dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<128>((const uint8_t *)sVt, 16 * ks, 32 * kk, lane),
                                                             dof[ks], dP, 0, 0, 0);
            }
            // keys past the item weigh 0; a query past the item (its lane clamped to the last row, so finite)
            // only feeds its own dQ row, which is not stored
            f32x16 dS;
            const int ulim = k1 - (kt + kk * 32 + 4 * hh);  // this lane's keys u = ... + 8 (r / 4) + r % 4
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = 8 * (r >> 2) + (r & 3) < ulim ? __builtin_amdgcn_exp2f(S[r] * kScale2 - lse2) : 0.f;
                dS[r] = p * (dP[r] - dlt);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 b = pack8(dS, s);
#pragma unroll
                for (int te = 0; te < 2; ++te)
                    dQ[te] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        tr_rows_frag((const uint8_t *)sK, kk * 32 + 16 * s, 32 * te, lane), b, dQ[te], 0, 0, 0);
            }
        }
        }
    }
    if (active && qvalid) {
        const float2 *rb = a.rope ? a.rope + (int)a.pos[(size_t)t * 4] * 32 : nullptr;
#pragma unroll
        for (int te = 0; te < 2; ++te)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 32 * te + 8 * i + 4 * hh;
                float g[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) g[j] = dQ[te][4 * i + j] * 0.125f;
                if (rb) unrotate4(g, *(const f32x4 *)(rb + e / 2));
                *(u32x2 *)(a.dq + (size_t)t * a.ldd + head * 64 + e) = u32x2{pack2(g[0], g[1]), pack2(g[2], g[3])};
            }
    }
}

__global__ __launch_bounds__(512, 1) void k_attn_bwd_dkv(AttnBwdArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[4 * 1024];  // stage: Q tile 512 | dO tile 512 chunks
    __shared__ __attribute__((aligned(16))) float sld[4][2][64];     // stage: lse, delta of the tile's queries
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int head = logical / a.ntiles, ti = logical % a.ntiles;
    const int2 tile = a.tiles[ti];
    const int k0 = a.cu[tile.x], k1 = a.cu[tile.x + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int kbase = tile.y + wave * 32;
    const bool active = kbase < k1;
    const bool kvalid = kbase + l32 < k1;
    const int u = min(kbase + l32, k1 - 1);
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = __builtin_bit_cast(bf16x8, load16(a.k + (size_t)u * a.ldqk + head * 64 + ks * 16 + hh * 8));
        // v of key u, features 16 ks + 8 hh .. + 7, gathered from the feature-major vt
        uint16_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = a.vt[(size_t)(head * 64 + ks * 16 + hh * 8 + e) * a.ldvt + u];
        vf[ks] = __builtin_bit_cast(bf16x8, e8);
    }
    const int prow = tid >> 3, pc = swzb(prow, tid & 7);
    const float *lse = a.lse + (size_t)head * a.ldl, *dl = a.delta + (size_t)head * a.ldl;
    auto issue = [&](int tt, int buf) {
        const int row = min(k0 + tt * 64 + prow, k1 - 1);
        u32x4 *dst = smem + buf * 1024;
        lds_dma16(a.q + (size_t)row * a.ldqk + head * 64 + pc * 8, dst + wave * 64);
        lds_dma16(a.dout + (size_t)row * a.lddo + head * 64 + pc * 8, dst + 512 + wave * 64);
        if (tid < 128) {  // queries past the item get lse = +inf (weight 0) and delta 0; delta is kept negated
            const int r = tid & 63, t = k0 + tt * 64 + r;
            const bool ok = t < k1;
            sld[buf][tid >> 6][r] = (tid < 64) ? (ok ? lse[t] : INFINITY) : (ok ? -dl[t] : 0.f);
        }
    };
    f32x16 dK[2] = {f32x16{}, f32x16{}}, dV[2] = {f32x16{}, f32x16{}};
    // One 32-query slice (half qq of query tile tt) in two steps. scores: S = Q K^T and dP - delta =
    // dO V^T - delta, the subtraction done by starting the dP accumulator at -delta of each row.
    auto scores = [&](int tt, int qq, f32x16 &S, f32x16 &dP) {
        const u32x4 *sQ = smem + (tt & 3) * 1024, *sO = sQ + 512;
        const int row = qq * 32 + l32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 d4 = *(const f32x4 *)&sld[tt & 3][1][qq * 32 + 8 * i + 4 * hh];
            dP[4 * i] = d4.x, dP[4 * i + 1] = d4.y, dP[4 * i + 2] = d4.z, dP[4 * i + 3] = d4.w;
        }
        S = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = swzb(row, ks * 2 + hh);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sQ[row * 8 + ch]), kf[ks], S, 0, 0, 0);
            dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sO[row * 8 + ch]), vf[ks], dP, 0, 0,
                                                         0);
        }
    };
    // grads: P and dS = P (dP - delta), then dV^T += dO^T P and dK^T += Q^T dS
    auto grads = [&](int tt, int qq, const f32x16 &S, const f32x16 &dP) {
        const u32x4 *sQ = smem + (tt & 3) * 1024, *sO = sQ + 512;
        f32x16 P, dS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 l4 = *(const f32x4 *)&sld[tt & 3][0][qq * 32 + 8 * i + 4 * hh];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 4 * i + jj;
                const float p = __builtin_amdgcn_exp2f(S[r] * kScale2 - lv[jj]);
                P[r] = p;
                dS[r] = p * dP[r];
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 bp = pack8(P, s), bs = pack8(dS, s);
#pragma unroll
            for (int te = 0; te < 2; ++te) {
                dV[te] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    tr_rows_frag((const uint8_t *)sO, qq * 32 + 16 * s, 32 * te, lane), bp, dV[te], 0, 0, 0);
                dK[te] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    tr_rows_frag((const uint8_t *)sQ, qq * 32 + 16 * s, 32 * te, lane), bs, dK[te], 0, 0, 0);
            }
        }
    };
    const int ntile = (k1 - k0 + 63) >> 6;
    // query tiles in pairs over four buffers, one barrier per pair (as in the dQ kernel)
    auto next_pair = [&](int tp) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        if (tp + 2 < ntile) issue(tp + 2, (tp + 2) & 3);
        if (tp + 3 < ntile) issue(tp + 3, (tp + 3) & 3);
    };
    issue(0, 0);
    if (1 < ntile) issue(1, 1);
    // the slices of a pair in a pipeline: each slice's products are issued before the previous slice's
    // exponentials, which then run while the matrix cores work on them
    f32x16 Sa, dPa, Sb, dPb;
    int tp = 0;
    for (; tp + 1 < ntile; tp += 2) {
        next_pair(tp);
        if (!active) continue;
        scores(tp, 0, Sa, dPa);
        scores(tp, 1, Sb, dPb);
        grads(tp, 0, Sa, dPa);
        scores(tp + 1, 0, Sa, dPa);
        grads(tp, 1, Sb, dPb);
        scores(tp + 1, 1, Sb, dPb);
        grads(tp + 1, 0, Sa, dPa);
        grads(tp + 1, 1, Sb, dPb);
    }
    if (tp < ntile) {  // an odd last tile
        next_pair(tp);
        if (active) {
            scores(tp, 0, Sa, dPa);
            scores(tp, 1, Sb, dPb);
            grads(tp, 0, Sa, dPa);
            grads(tp, 1, Sb, dPb);
        }
    }
    if (active && kvalid) {
        const float2 *rb = a.rope ? a.rope + (int)a.pos[(size_t)u * 4] * 32 : nullptr;
#pragma unroll
        for (int te = 0; te < 2; ++te)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 32 * te + 8 * i + 4 * hh;
                float g[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) g[j] = dK[te][4 * i + j] * 0.125f;
                if (rb) unrotate4(g, *(const f32x4 *)(rb + e / 2));
                *(u32x2 *)(a.dk + (size_t)u * a.ldd + head * 64 + e) = u32x2{pack2(g[0], g[1]), pack2(g[2], g[3])};
                *(u32x2 *)(a.dv + (size_t)u * a.ldd + head * 64 + e) =
                    u32x2{pack2(dV[te][4 * i], dV[te][4 * i + 1]), pack2(dV[te][4 * i + 2], dV[te][4 * i + 3])};
            }
    }
}

// one thread per (token, 8 features): gate and up are interleaved in blocks of 32 features, so the 8
// gates, the 8 ups, their 8 output gradients and the 8 activations are each one 16-byte access. SiLU as in
// the forward's epilogue: s = 1 / (1 + 2^(-g log2 e)) on the raw v_exp_f32 and v_rcp_f32.
__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t *gu, const uint16_t *da, uint16_t *dgu, uint16_t *a,
                                                    int T, int F) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * (F / 8)) return;
    const int t = (int)(idx / (F / 8)), f = (int)(idx % (F / 8)) * 8;
    const int blk = f >> 5, w = f & 31;
    const size_t gi = (size_t)t * 2 * F + blk * 64 + w, ui = gi + 32, ai = (size_t)t * F + f;
    const u32x4 gg = *(const u32x4 *)(gu + gi), uu = *(const u32x4 *)(gu + ui), dd = *(const u32x4 *)(da + ai);
    const uint32_t g2[4] = {gg.x, gg.y, gg.z, gg.w}, u2[4] = {uu.x, uu.y, uu.z, uu.w}, d2[4] = {dd.x, dd.y, dd.z, dd.w};
    uint32_t dg[4], du[4], av[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float o[3][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float g = bf16_to_f32(h ? g2[q] >> 16 : g2[q] & 0xffff);
            const float up = bf16_to_f32(h ? u2[q] >> 16 : u2[q] & 0xffff);
            const float d = bf16_to_f32(h ? d2[q] >> 16 : d2[q] & 0xffff);
            const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
            const float silu = g * sg;
            o[0][h] = d * up * sg * (1.f + g * (1.f - sg));  // d/dg
            o[1][h] = d * silu;                             // d/du
            o[2][h] = silu * up;                            // the activation
        }
        dg[q] = pack2(o[0][0], o[0][1]), du[q] = pack2(o[1][0], o[1][1]), av[q] = pack2(o[2][0], o[2][1]);
    }
    *(u32x4 *)(dgu + gi) = u32x4{dg[0], dg[1], dg[2], dg[3]};
    *(u32x4 *)(dgu + ui) = u32x4{du[0], du[1], du[2], du[3]};
    *(u32x4 *)(a + ai) = u32x4{av[0], av[1], av[2], av[3]};
}

// One wave per row; workgroup (4 waves) = rows_per_block consecutive rows, so the gain partial of the
// block is summed in a fixed order. Lane l holds columns 64 V c + V l .. + V - 1 (c < D / 64 V) and moves
// them with V-wide loads and stores; each wave keeps two rows in flight.
template <int V, int CM>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const float *x, const float *gain, const float *dh,
                                                     const float *dres, float *dx, uint16_t *dxb, float *gpart,
                                                     int rows_per_block, int T, int D, float eps) {
    __shared__ float sg[4][1024];
    typedef float fv __attribute__((ext_vector_type(V)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int C = CM;  // column groups: D = 64 V CM
    float gacc[CM][V], gv[CM][V];
#pragma unroll
    for (int c = 0; c < CM; ++c)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            gacc[c][v] = 0.f;
            gv[c][v] = c < C ? gain[64 * V * c + V * lane + v] : 0.f;
        }
    const int r0 = blockIdx.x * rows_per_block, r1 = min(T, r0 + rows_per_block);
    auto row = [&](int t, const fv (&xv)[CM], const fv (&hv)[CM], const fv (&rv)[CM]) {
        float ss = 0.f, sd = 0.f;
#pragma unroll
        for (int c = 0; c < CM; ++c)
            if (c < C)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    ss += xv[c][v] * xv[c][v];
                    sd += hv[c][v] * gv[c][v] * xv[c][v];
                }
        ss = wave_sum(ss);
        sd = wave_sum(sd);
        const float inv = 1.0f / sqrtf(ss / (float)D + eps);
        const float k = inv * inv * inv * sd / (float)D;
#pragma unroll
        for (int c = 0; c < CM; ++c)
            if (c < C) {
                const size_t i = (size_t)t * D + 64 * V * c + V * lane;
                fv o;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    o[v] = inv * gv[c][v] * hv[c][v] - xv[c][v] * k;
                    gacc[c][v] += hv[c][v] * xv[c][v] * inv;
                }
                if (dres) o += rv[c];
                *(fv *)(dx + i) = o;
                if (dxb) {
                    if constexpr (V == 4)
                        *(u32x2 *)(dxb + i) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                    else
                        *(uint32_t *)(dxb + i) = pack2(o[0], o[1]);
                }
            }
    };
    // x, dh and the residual gradient of a row are loaded together (dres joins them rather than waiting for
    // the row's reductions)
    auto load = [&](int t, fv (&xv)[CM], fv (&hv)[CM], fv (&rv)[CM]) {
#pragma unroll
        for (int c = 0; c < CM; ++c)
            if (c < C) {
                const size_t i = (size_t)t * D + 64 * V * c + V * lane;
                xv[c] = *(const fv *)(x + i);
                hv[c] = *(const fv *)(dh + i);
                rv[c] = dres ? *(const fv *)(dres + i) : fv{};
            }
    };
    int t = r0 + wave;
    for (; t + 4 < r1; t += 8) {
        fv xa[CM], ha[CM], ra[CM], xb[CM], hb[CM], rb[CM];
        load(t, xa, ha, ra);
        load(t + 4, xb, hb, rb);
        row(t, xa, ha, ra);
        row(t + 4, xb, hb, rb);
    }
    if (t < r1) {
        fv xa[CM], ha[CM], ra[CM];
        load(t, xa, ha, ra);
        row(t, xa, ha, ra);
    }
#pragma unroll
    for (int c = 0; c < CM; ++c)
        if (c < C)
#pragma unroll
            for (int v = 0; v < V; ++v) sg[wave][64 * V * c + V * lane + v] = gacc[c][v];
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += 256) gpart[(size_t)blockIdx.x * D + i] = ((sg[0][i] + sg[1][i]) + sg[2][i]) + sg[3][i];
}

// Column sums in two fixed-order levels: slices of kColSlice rows into partials (one thread per column and
// slice), then the partials of a column in slice order. `square`: sum g^2 + eps1 instead of g.
constexpr int kColSlice = 32;

__global__ __launch_bounds__(256) void k_col_parts(const float *src, int rows, int cols, float *parts, int square,
                                                   float eps1) {
    const int j = blockIdx.x * 256 + threadIdx.x, sl = blockIdx.y;
    if (j >= cols) return;
    const int r0 = sl * kColSlice, r1 = min(rows, r0 + kColSlice);
    float s = 0.f;
    for (int i = r0; i < r1; ++i) {
        const float v = src[(size_t)i * cols + j];
        s += square ? v * v + eps1 : v;
    }
    parts[(size_t)sl * cols + j] = s;
}

__global__ __launch_bounds__(256) void k_sum_rows(const float *part, int blocks, int D, float *out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= D) return;
    float s = 0.f;
    for (int b = 0; b < blocks; ++b) s += part[(size_t)b * D + i];
    out[i] = s;
}

// ------------------------------------------------------------------------------------ weight gradients
//
// out[m][n] = sum over t of X[t][m] Y[t][n]. Workgroup tile 64 n x 128 m, 4 waves (32 m each, two 32x32
// MFMA tiles along n): C = Y^T X, A operand = Y^T (rows n) and B = X (columns m), both read k-major (k = t)
// through the transpose load from LDS tiles of 64 tokens; a lane ends with 4 consecutive n of one m, so the
// fp32 partials are stored as rows of out. Split over t into `splits` ranges of `chunk` tokens (a multiple
// of 64); the last range's rows past T are zeroed in LDS.
constexpr int kXtyStage = 512 + 1024;  // chunks: Y tile [64 t][64 n] | X tile [64 t][128 m]
constexpr int kXtyLoads = 2 + 4;       // DMA loads per thread per stage (Y rounds + X rounds)

__global__ __launch_bounds__(256, 2) void k_xty(const uint16_t *x, int ldx, const uint16_t *y, int ldy, int T, int M,
                                                int N, float *partial, int chunk) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[2 * kXtyStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int MT = M / 128, NT = N / 64;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int s = logical / (MT * NT), rest = logical % (MT * NT);
    const int mt = rest / NT, nt = rest % NT;  // consecutive tiles share their X columns
    const int m0 = mt * 128, n0 = nt * 64;
    const int tb = s * chunk, te = min(T, tb + chunk);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    const int yrow = tid >> 3, ych = tid & 7;    // Y tile: 64 rows x 8 chunks, 2 rounds of 32 rows
    const int xrow = tid >> 4, xch = tid & 15;   // X tile: 64 rows x 16 chunks, 4 rounds of 16 rows
    auto issue = [&](int t0, int buf) {
        u32x4 *st = smem + buf * kXtyStage;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 32 * r + yrow, src = min(t0 + row, T - 1);
            lds_dma16(y + (size_t)src * ldy + n0 + ((ych ^ kmajor_swz<128>(row)) << 3), st + r * 256 + wave * 64);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * r + xrow, src = min(t0 + row, T - 1);
            lds_dma16(x + (size_t)src * ldx + m0 + ((xch ^ kmajor_swz<256>(row)) << 3), st + 512 + r * 256 + wave * 64);
        }
    };
    const int nk = te > tb ? (te - tb + 63) >> 6 : 0;
    // The next stage's DMA is issued before this stage's wait (its buffer was freed by the previous
    // iteration's closing barrier), so it has a whole stage of compute and both barriers to land.
    if (nk) issue(tb, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1, t0 = tb + kt * 64;
        if (kt + 1 < nk) {
            issue(t0 + 64, buf ^ 1);
            wait_vmcnt<kXtyLoads>();  // this stage's loads are the older ones
        } else {
            wait_vmcnt<0>();
        }
        if (t0 + 64 > te) {  // rows past the range read as zero
            u32x4 *st = smem + buf * kXtyStage;
#pragma unroll
            for (int r = 0; r < 2; ++r)
                if (t0 + 32 * r + yrow >= te) st[r * 256 + tid] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (t0 + 16 * r + xrow >= te) st[512 + r * 256 + tid] = u32x4{0u, 0u, 0u, 0u};
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        const uint8_t *sY = (const uint8_t *)(smem + buf * kXtyStage), *sX = sY + 512 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 b = tr_frag<256>(sX, 16 * ks, 32 * wave, lane);
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
                acc[tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<128>(sY, 16 * ks, 32 * tn, lane), b, acc[tn], 0, 0, 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
    }
    const int m = m0 + 32 * wave + l32;
    float *out = partial + ((size_t)s * M + m) * N + n0 + 4 * hh;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(f32x4 *)(out + 32 * tn + 8 * i) = f32x4{acc[tn][4 * i], acc[tn][4 * i + 1], acc[tn][4 * i + 2], acc[tn][4 * i + 3]};
}

// The same product for M % 256 == 0 and N % 256 == 0: a 256 n x 256 m tile per workgroup of 8 waves;
// wave (wn = wave % 2, wm = wave / 2) holds n rows 128 wn .. + 127 (four 32-row A tiles of Y^T) against m
// columns 64 wm .. + 63 (two 32-column B tiles of X). LDS stages of 64 tokens hold both tiles as 512-byte
// rows (chunks swizzled by 4 (t % 4), which keeps the transpose reads of a 16-lane group on distinct banks);
// two stages, the next one's DMA in flight during the current one's products.
constexpr int kXtyWideStage = 2 * 2048;  // 16-byte chunks: Y tile [64 t][256 n] | X tile [64 t][256 m]
constexpr int kXtyWideLoads = 4 + 4;     // DMA loads per thread per stage (Y rounds + X rounds)

__global__ __launch_bounds__(512, 1) void k_xty256(const uint16_t *x, int ldx, const uint16_t *y, int ldy, int T,
                                                   int M, int N, float *partial, int chunk) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[2 * kXtyWideStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int wn = wave & 1, wm = wave >> 1;
    const int MT = M / 256, NT = N / 256;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int s = logical / (MT * NT), rest = logical % (MT * NT);
    const int mt = rest / NT, nt = rest % NT;  // consecutive tiles share their X columns
    const int m0 = mt * 256, n0 = nt * 256;
    const int tb = s * chunk, te = min(T, tb + chunk);
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x16{};
    const int lrow = tid >> 5, lch = tid & 31;  // 16 rows of 32 chunks per round, 4 rounds per tile
    auto issue = [&](int t0, int buf) {
        u32x4 *st = smem + buf * kXtyWideStage;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * r + lrow, src = min(t0 + row, T - 1);
            lds_dma16(y + (size_t)src * ldy + n0 + ((lch ^ kmajor_swz<512>(row)) << 3), st + r * 512 + wave * 64);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * r + lrow, src = min(t0 + row, T - 1);
            lds_dma16(x + (size_t)src * ldx + m0 + ((lch ^ kmajor_swz<512>(row)) << 3),
                      st + 2048 + r * 512 + wave * 64);
        }
    };
    const int nk = te > tb ? (te - tb + 63) >> 6 : 0;
    // The next stage's DMA is issued before this stage's wait (its buffer was freed by the previous
    // iteration's closing barrier), so it has a whole stage of compute and both barriers to land.
    if (nk) issue(tb, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1, t0 = tb + kt * 64;
        if (kt + 1 < nk) {
            issue(t0 + 64, buf ^ 1);
            wait_vmcnt<kXtyWideLoads>();  // this stage's loads are the older ones
        } else {
            wait_vmcnt<0>();
        }
        if (t0 + 64 > te) {  // rows past the range read as zero
            u32x4 *st = smem + buf * kXtyWideStage;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (t0 + 16 * r + lrow >= te) {
                    st[r * 512 + tid] = u32x4{0u, 0u, 0u, 0u};
                    st[2048 + r * 512 + tid] = u32x4{0u, 0u, 0u, 0u};
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        const uint8_t *sY = (const uint8_t *)(smem + buf * kXtyWideStage), *sX = sY + 2048 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 b0 = tr_frag<512>(sX, 16 * ks, 64 * wm, lane);
            const bf16x8 b1 = tr_frag<512>(sX, 16 * ks, 64 * wm + 32, lane);
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const bf16x8 a = tr_frag<512>(sY, 16 * ks, 128 * wn + 32 * tn, lane);
                acc[tn][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[tn][0], 0, 0, 0);
                acc[tn][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[tn][1], 0, 0, 0);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
        const int m = m0 + 64 * wm + 32 * tm + l32;
        float *out = partial + ((size_t)s * M + m) * N + n0 + 128 * wn + 4 * hh;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(f32x4 *)(out + 32 * tn + 8 * i) = f32x4{acc[tn][tm][4 * i], acc[tn][tm][4 * i + 1],
                                                          acc[tn][tm][4 * i + 2], acc[tn][tm][4 * i + 3]};
    }
}

// four consecutive outputs per thread (M * N % 4 == 0; a group of four never straddles a 32-column block)
__global__ __launch_bounds__(256) void k_xty_reduce(const float *partial, int splits, int M, int N, float *out,
                                                    float *out2, int deinterleave) {
    const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (idx >= (size_t)M * N) return;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) s += *(const f32x4 *)(partial + (size_t)sp * M * N + idx);
    if (!deinterleave) {
        *(f32x4 *)(out + idx) = s;
        return;
    }
    const int m = (int)(idx / N), n = (int)(idx % N);
    const int blk = n >> 6, w = n & 63, half = N / 2;
    if (w < 32) *(f32x4 *)(out + (size_t)m * half + blk * 32 + w) = s;
    else *(f32x4 *)(out2 + (size_t)m * half + blk * 32 + w - 32) = s;
}

// -------------------------------------------------------------------------------- embedding and pool

// one workgroup per byte value: its tokens' gradient rows summed in token order
// One workgroup (8 waves) per byte value: wave w sums the rows of the w-th eighth of that value's tokens
// (token order; lane l holds columns 4 l + 256 g .. + 3), then the eight partial rows are added in wave
// order.
__global__ __launch_bounds__(512) void k_embed_bwd(const float *dx, const uint32_t *tok_off, const uint32_t *tok, int D,
                                                   float *dE) {
    __shared__ __attribute__((aligned(16))) float part[8][1024];
    const int v = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t p0 = tok_off[v], n = tok_off[v + 1] - p0;
    const uint32_t q0 = p0 + (uint32_t)((uint64_t)n * wave / 8), q1 = p0 + (uint32_t)((uint64_t)n * (wave + 1) / 8);
    f32x4 acc[4] = {};
    for (uint32_t p = q0; p < q1; ++p) {
        const float *row = dx + (size_t)tok[p] * D;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = 256 * g + 4 * lane;
            if (c < D) acc[g] += *(const f32x4 *)(row + c);
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int c = 256 * g + 4 * lane;
        if (c < D) *(f32x4 *)&part[wave][c] = acc[g];
    }
    __syncthreads();
    for (int i = tid; i < D; i += 512) {
        float sum = part[0][i];
        for (int w = 1; w < 8; ++w) sum += part[w][i];
        dE[(size_t)v * D + i] = sum;
    }
}

// Pool backward. With p = softmax over an item's tokens of s_t,h, z_h = sum_t p_t,h xf_t and
// pooled_h = z_h W_v,h (W_v,h = columns 64h .. 64h + 63 of W_v):
//   dz_h = W_v,h dpooled_h;  a_t,h = xf_t . dz_h;  ds_t,h = p_t,h (a_t,h - sum_t p a);
//   dxf_t = sum_h (p_t,h dz_h + ds_t,h u_h);  du_h = sum over items and tokens of ds_t,h xf_t;
//   dW_v[:, 64h + e] = sum over items of z_h dpooled_h[e];  u_h = W_k,h q_h / 8 gives
//   dW_k[:, 64h + e] = du_h q_h[e] / 8 and dq_h[e] = W_k[:, 64h + e] . du_h / 8.
// Every sum runs in a fixed order (tokens ascending, items ascending).

// dz[item][h][i], one thread per (h, i)
__global__ __launch_bounds__(256) void k_pool_bwd_dz(PoolBwdArgs a, float *dz) {
    const int item = blockIdx.y, x = blockIdx.x * 256 + threadIdx.x;
    if (x >= a.H * a.D) return;
    const int h = x / a.D, i = x % a.D;
    float s = 0.f;
    for (int e = 0; e < 64; ++e) s += bf16_to_f32(a.wv[(size_t)i * a.D + 64 * h + e]) * a.dpooled[(size_t)item * a.D + 64 * h + e];
    dz[((size_t)item * a.H + h) * a.D + i] = s;
}

// p and a of every (token, head) into pd[t][h][2] and sum_t p a per (item, head) into spa; one workgroup
// (8 waves) per item. Softmax statistics per head by a fixed tree over the threads; then wave w takes the
// item's tokens t0 + w, t0 + w + 8, ...: lane l holds columns 8 l + 512 c .. + 7 (c < CG) of xf_t and of
// dz_h for 8 heads at a time, a_t,h = xf_t . dz_h comes from a cross-lane tree (head h ends in lanes
// 8h .. 8h + 7), and those lanes keep p_t,h and the running sum of p a (token order per wave, then the
// waves in order).
template <int CG>
__global__ __launch_bounds__(512) void k_pool_bwd_tokens(PoolBwdArgs a, const float *dz, float *pd, float *spa,
                                                         int tchunks) {
    __shared__ float red[8][16];
    __shared__ float mh[16], ih[16];
    const int item = blockIdx.x, ch = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D, H = a.H, t0 = a.cu[item], t1 = a.cu[item + 1];
    float *spa_out = spa + ((size_t)item * tchunks + ch) * H;  // this token range's sums of p a
    if (t1 == t0) {
        if (tid < H) spa_out[tid] = 0.f;
        return;
    }
    // this workgroup's range of the item's tokens (statistics still over the whole item)
    const int len = t1 - t0;
    const int r0 = t0 + (int)((long long)len * ch / tchunks), r1 = t0 + (int)((long long)len * (ch + 1) / tchunks);
    // softmax statistics of every head
    float loc[16];
#pragma unroll
    for (int hd = 0; hd < 16; ++hd) loc[hd] = -INFINITY;
    for (int t = t0 + tid; t < t1; t += 512)
#pragma unroll
        for (int hd = 0; hd < 16; ++hd)
            if (hd < H) loc[hd] = fmaxf(loc[hd], a.s[(size_t)t * H + hd]);
#pragma unroll
    for (int hd = 0; hd < 16; ++hd) {
        const float v = wave_max(loc[hd]);
        if (lane == 0 && hd < H) red[wave][hd] = v;
    }
    __syncthreads();
    if (tid < H) {
        float m = red[0][tid];
        for (int w = 1; w < 8; ++w) m = fmaxf(m, red[w][tid]);
        mh[tid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hd = 0; hd < 16; ++hd) loc[hd] = 0.f;
    for (int t = t0 + tid; t < t1; t += 512)
#pragma unroll
        for (int hd = 0; hd < 16; ++hd)
            if (hd < H) loc[hd] += __expf(a.s[(size_t)t * H + hd] - mh[hd]);
#pragma unroll
    for (int hd = 0; hd < 16; ++hd) {
        const float v = wave_sum(loc[hd]);
        if (lane == 0 && hd < H) red[wave][hd] = v;
    }
    __syncthreads();
    if (tid < H) {
        float sum = red[0][tid];
        for (int w = 1; w < 8; ++w) sum += red[w][tid];
        ih[tid] = 1.0f / sum;
    }
    __syncthreads();
    for (int h0 = 0; h0 < H; h0 += 8) {
        float dzr[CG][8][8];
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int hd = 0; hd < 8; ++hd)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int col = 512 * c + 8 * lane + i;
                    dzr[c][hd][i] = (h0 + hd < H && col < D) ? dz[((size_t)item * H + h0 + hd) * D + col] : 0.f;
                }
        const int hl = h0 + (lane >> 3);  // the head whose total this lane receives
        const bool mine = hl < H;
        const float mhl = mine ? mh[hl] : 0.f, ihl = mine ? ih[hl] : 0.f;
        float pa = 0.f;
        auto tok = [&](int t, const u32x4 (&v)[CG]) {
            float d[8];
#pragma unroll
            for (int hd = 0; hd < 8; ++hd) d[hd] = 0.f;
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const uint32_t w4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x0 = bf16_to_f32(w4[q] & 0xffff), x1 = bf16_to_f32(w4[q] >> 16);
#pragma unroll
                    for (int hd = 0; hd < 8; ++hd) d[hd] += x0 * dzr[c][hd][2 * q] + x1 * dzr[c][hd][2 * q + 1];
                }
            }
            const float av = lanes_reduce<8>(d, lane);
            if (mine) {
                const float p = __expf(a.s[(size_t)t * H + hl] - mhl) * ihl;
                pa += p * av;
                if ((lane & 7) == 0) *(float2 *)(pd + ((size_t)t * H + hl) * 2) = float2{p, av};
            }
        };
        auto load = [&](int t, u32x4 (&v)[CG]) {
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const int col = 512 * c + 8 * lane;
                v[c] = col < D ? *(const u32x4 *)(a.xf + (size_t)t * D + col) : u32x4{0u, 0u, 0u, 0u};
            }
        };
        int t = r0 + wave;
        for (; t + 24 < r1; t += 32) {
            u32x4 v[4][CG];
#pragma unroll
            for (int k = 0; k < 4; ++k) load(t + 8 * k, v[k]);
#pragma unroll
            for (int k = 0; k < 4; ++k) tok(t + 8 * k, v[k]);
        }
        for (; t < r1; t += 8) {
            u32x4 v[CG];
            load(t, v);
            tok(t, v);
        }
        __syncthreads();
        if ((lane & 7) == 0 && mine) red[wave][hl - h0] = pa;
        __syncthreads();
        if (tid < 8 && h0 + tid < H) {
            float sum = red[0][tid];
            for (int w = 1; w < 8; ++w) sum += red[w][tid];
            spa_out[h0 + tid] = sum;
        }
    }
}

// One workgroup per (256 columns, item, range of the item's tokens), one thread per column: per token
// ds_h = p_h (a_h - spa_h) and dxf_t = sum_h (p_h dz_h + ds_h u_h); the range's partial sums of
// z_h = sum p x and du_h = sum ds x (token order).
__global__ __launch_bounds__(256) void k_pool_bwd_cols(PoolBwdArgs a, const float *dz, const float *pd,
                                                       const float *spa, int tchunks, float *zpart, float *dupart,
                                                       int chunks) {
    const int item = blockIdx.y, ch = blockIdx.z, i = blockIdx.x * 256 + threadIdx.x;
    const int D = a.D, H = a.H, t0 = a.cu[item], t1 = a.cu[item + 1];
    if (i >= D) return;
    const int len = t1 - t0;
    const int c0 = t0 + (int)((long long)len * ch / chunks), c1 = t0 + (int)((long long)len * (ch + 1) / chunks);
    float dzv[16], uv[16], sp[16], zv[16], duv[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        zv[h] = duv[h] = 0.f;
        dzv[h] = h < H ? dz[((size_t)item * H + h) * D + i] : 0.f;
        uv[h] = h < H ? a.u[(size_t)h * D + i] : 0.f;
        sp[h] = 0.f;
        for (int c = 0; c < tchunks; ++c) sp[h] += h < H ? spa[((size_t)item * tchunks + c) * H + h] : 0.f;
    }
    for (int t = c0; t < c1; ++t) {
        const float xv = bf16_to_f32(a.xf[(size_t)t * D + i]);
        float g = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            if (h < H) {
                const float2 q = *(const float2 *)(pd + ((size_t)t * H + h) * 2);
                const float ds = q.x * (q.y - sp[h]);
                zv[h] += q.x * xv;
                duv[h] += ds * xv;
                g += q.x * dzv[h] + ds * uv[h];
            }
        }
        a.dxf[(size_t)t * D + i] = g;
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        if (h < H) {
            const size_t o = (((size_t)item * chunks + ch) * H + h) * D + i;
            zpart[o] = zv[h];
            dupart[o] = duv[h];
        }
    }
}

// per item: z and du from the ranges' partials (ranges ascending), one thread per (h, i)
__global__ __launch_bounds__(256) void k_pool_bwd_item_sums(PoolBwdArgs a, const float *zpart, const float *dupart,
                                                            int chunks) {
    const int item = blockIdx.y, x = blockIdx.x * 256 + threadIdx.x, HD = a.H * a.D;
    if (x >= HD) return;
    float zs = 0.f, ds = 0.f;
    for (int ch = 0; ch < chunks; ++ch) {
        const size_t o = ((size_t)item * chunks + ch) * HD + x;
        zs += zpart[o];
        ds += dupart[o];
    }
    a.z[(size_t)item * HD + x] = zs;
    a.du[(size_t)item * HD + x] = ds;
}

// du totals over items (items ascending), one thread per (h, i)
__global__ __launch_bounds__(256) void k_pool_bwd_du(PoolBwdArgs a, float *du_tot) {
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x >= a.H * a.D) return;
    float s = 0.f;
    for (int item = 0; item < a.count; ++item) s += a.du[(size_t)item * a.H * a.D + x];
    du_tot[x] = s;
}

// weight gradients, one thread per (i, column c = 64h + e) of dW_v and dW_k; one thread per c of dq
__global__ __launch_bounds__(256) void k_pool_bwd_weights(PoolBwdArgs a, const float *du_tot) {
    const int D = a.D, H = a.H;
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x < (size_t)D * D) {
        const int i = (int)(x / D), c = (int)(x % D), h = c / 64;
        float wv = 0.f;
        for (int item = 0; item < a.count; ++item)
            wv += a.z[((size_t)item * H + h) * D + i] * a.dpooled[(size_t)item * D + c];
        a.dwv[x] = wv;
        a.dwk[x] = du_tot[(size_t)h * D + i] * bf16_to_f32(a.query[c]) * 0.125f;
    } else if (x < (size_t)D * D + (size_t)D * 64) {
        // one wave per query column c: lane l sums rows l, l + 64, ..., then a fixed tree over the lanes
        const int c = (int)((x - (size_t)D * D) >> 6), l = (int)(x & 63), h = c / 64;
        float dq = 0.f;
        for (int r = l; r < D; r += 64) dq += bf16_to_f32(a.wk[(size_t)r * D + c]) * du_tot[(size_t)h * D + r];
        dq = wave_sum(dq);
        if (l == 0) a.dquery[c] = dq * 0.125f;
    }
}

// ------------------------------------------------------------------------------------------ Adafactor
//
// Shazeer and Stern's update with the first moment the pages add, over the gradient cast to bf16: for a matrix, row and column means of
// g^2 + eps1 decayed by beta2 (r, c), v = r c^T / mean(r); for a vector, v decayed elementwise;
// u = g / sqrt(v), clipped to RMS(u) <= clip; m = beta1 m + (1 - beta1) u; w -= lr m / (1 - beta1^t).
// Every tensor of the model in the same four launches (statistics, column means, sums of u^2, update);
// a workgroup finds its tensor by binary search over the table's first-workgroup fields. Sums run over
// fixed ranges in a fixed order.

template <int kField>
__device__ __forceinline__ int ada_first(const AdaTensor &t) {
    return kField == 0 ? t.wg_stats : (kField == 1 ? t.wg_cols : t.wg_upd);
}

// the last tensor whose first workgroup (of grid kField) is <= wg
template <int kField>
__device__ int ada_find(const AdaTensor *tab, int n, int wg) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ada_first<kField>(tab[mid]) <= wg) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float block_sum256(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

// the optimizer reads each fp32 gradient cast to bf16 (round to nearest even)
__device__ __forceinline__ float ada_grad(const AdaTensor &a, size_t idx) {
    return bf16_to_f32(f32_to_bf16(a.g[idx]));
}

// matrices: one workgroup per slice of kAdaSlice rows (column partials of the slice, then the decayed
// row means); vectors: 256 elements of v per workgroup
__global__ __launch_bounds__(256) void k_ada_stats(const AdaTensor *tab, int n, AdaStep st) {
    const int t = ada_find<0>(tab, n, blockIdx.x);
    const AdaTensor a = tab[t];
    const int local = blockIdx.x - a.wg_stats, tid = threadIdx.x;
    if (a.cols == 0) {
        const int i = local * 256 + tid;
        if (i < a.rows) {
            const float g = ada_grad(a, i);
            a.v[i] = st.beta2 * a.v[i] + (1.f - st.beta2) * (g * g + st.eps1);
        }
        return;
    }
    const int r0 = local * kAdaSlice, r1 = min(a.rows, r0 + kAdaSlice);
    for (int j = tid; j < a.cols; j += 256) {
        float sum = 0.f;
        for (int i = r0; i < r1; ++i) {
            const float g = ada_grad(a, (size_t)i * a.cols + j);
            sum += g * g + st.eps1;
        }
        a.col_parts[(size_t)local * a.cols + j] = sum;
    }
    const int lane = tid & 63, wave = tid >> 6;
    for (int k = 0; k < kAdaSlice / 4; ++k) {
        const int row = r0 + wave * (kAdaSlice / 4) + k;
        if (row >= r1) break;
        float sum = 0.f;
        for (int j = lane; j < a.cols; j += 64) {
            const float g = ada_grad(a, (size_t)row * a.cols + j);
            sum += g * g + st.eps1;
        }
        sum = wave_sum(sum);
        if (lane == 0) a.r[row] = st.beta2 * a.r[row] + (1.f - st.beta2) * sum / (float)a.cols;
    }
}

// matrices: decayed column means from the slice partials (slice order), 256 columns per workgroup; the
// tensor's first workgroup also writes mean(r)
__global__ __launch_bounds__(256) void k_ada_cols(const AdaTensor *tab, int n, AdaStep st) {
    __shared__ float red[4];
    const int t = ada_find<1>(tab, n, blockIdx.x);
    const AdaTensor a = tab[t];
    const int local = blockIdx.x - a.wg_cols, tid = threadIdx.x;
    if (local == 0) {
        float sum = 0.f;
        for (int i = tid; i < a.rows; i += 256) sum += a.r[i];
        sum = block_sum256(sum, red);
        if (tid == 0) a.mean_r[0] = sum / (float)a.rows;
    }
    const int j = local * 256 + tid;
    if (j >= a.cols) return;
    const int slices = (a.rows + kAdaSlice - 1) / kAdaSlice;
    float sum = 0.f;
    for (int b = 0; b < slices; ++b) sum += a.col_parts[(size_t)b * a.cols + j];
    a.c[j] = st.beta2 * a.c[j] + (1.f - st.beta2) * sum / (float)a.rows;
}

__device__ __forceinline__ float ada_u(const AdaTensor &a, int idx, float mean_r) {
    const float g = ada_grad(a, idx);
    if (a.cols == 0) return g * rsqrtf(a.v[idx]);
    const int i = idx / a.cols, j = idx - i * a.cols;
    return g * rsqrtf(a.r[i] * a.c[j] / mean_r);
}

// sum of u^2 over each chunk of kAdaChunk elements
__global__ __launch_bounds__(256) void k_ada_rms(const AdaTensor *tab, int n, AdaStep st) {
    __shared__ float red[4];
    const int t = ada_find<2>(tab, n, blockIdx.x);
    const AdaTensor a = tab[t];
    const int local = blockIdx.x - a.wg_upd;
    const int count = a.rows * (a.cols ? a.cols : 1);
    const int e0 = local * kAdaChunk, e1 = min(count, e0 + kAdaChunk);
    const float mean_r = a.cols ? a.mean_r[0] : 1.f;
    float sum = 0.f;
    for (int x = e0 + threadIdx.x; x < e1; x += 256) {
        const float u = ada_u(a, x, mean_r);
        sum += u * u;
    }
    sum = block_sum256(sum, red);
    if (threadIdx.x == 0) a.rms_parts[local] = sum;
}

// clip factor from all chunks' sums, then the first moment and the master update of this chunk
__global__ __launch_bounds__(256) void k_ada_apply(const AdaTensor *tab, int n, AdaStep st) {
    __shared__ float red[4];
    const int t = ada_find<2>(tab, n, blockIdx.x);
    const AdaTensor a = tab[t];
    const int local = blockIdx.x - a.wg_upd;
    const int count = a.rows * (a.cols ? a.cols : 1);
    const int chunks = (count + kAdaChunk - 1) / kAdaChunk;
    float sum = 0.f;
    for (int b = threadIdx.x; b < chunks; b += 256) sum += a.rms_parts[b];
    sum = block_sum256(sum, red);
    const float rms = sqrtf(sum / (float)count);
    const float scale = 1.f / fmaxf(1.f, rms / st.clip);
    const float mean_r = a.cols ? a.mean_r[0] : 1.f;
    const int e0 = local * kAdaChunk, e1 = min(count, e0 + kAdaChunk);
    for (int x = e0 + threadIdx.x; x < e1; x += 256) {
        const float u = ada_u(a, x, mean_r) * scale;
        const float m = st.beta1 * a.m[x] + (1.f - st.beta1) * u;
        a.m[x] = m;
        const float step = st.lr * m / st.bias_correction;
        if (a.w16) a.w16[x] = (uint16_t)f32_to_bf16(bf16_to_f32(a.w16[x]) - step);
        else a.w32[x] = a.w32[x] - step;
    }
}

// -------------------------------------------------------------------------------------------- packing
//
// The forward's and the backward's derived copies of the masters, every one in one launch: a table of
// jobs, each a range of workgroups (binary search over first_wg).

__device__ int pack_find(const PackJob *jobs, int n, int wg) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].first_wg <= wg) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_pack(const PackJob *jobs, int n) {
    __shared__ float tile[64][65];
    const PackJob jb = jobs[pack_find(jobs, n, blockIdx.x)];
    const int local = blockIdx.x - jb.first_wg, tid = threadIdx.x;
    const int K = jb.K, N = jb.N;
    if (jb.kind == kPackTranspose || jb.kind == kPackTransposePair) {
        // out[n][k] = bf16(W[k][n] * gain[k]) through a 64 x 64 LDS tile; pair: out row n takes column
        // 32 (n / 64) + n % 32 of W (n % 64 < 32) or of W2
        const bool pair = jb.kind == kPackTransposePair;
        const int NO = pair ? 2 * N : N, ntn = (NO + 63) / 64;
        const int n0 = (local % ntn) * 64, k0 = (local / ntn) * 64;
        const uint16_t *w = (const uint16_t *)jb.src, *w2 = (const uint16_t *)jb.src2;
        for (int x = tid; x < 64 * 64; x += 256) {
            const int kk = x >> 6, nn = x & 63, nx = n0 + nn;
            const uint16_t *src = w;
            int col = nx;
            if (pair) {
                src = (nx & 63) < 32 ? w : w2;
                col = (nx >> 6) * 32 + (nx & 31);
            }
            const bool in = nx < NO && k0 + kk < K;
            const float g = jb.gain && in ? jb.gain[k0 + kk] : 1.f;
            tile[kk][nn] = in ? bf16_to_f32(src[(size_t)(k0 + kk) * N + col]) * g : 0.f;
        }
        __syncthreads();
        uint16_t *out = (uint16_t *)jb.dst;
        for (int x = tid; x < 64 * 64; x += 256) {
            const int nn = x >> 6, kk = x & 63;
            if (n0 + nn < NO && k0 + kk < K) out[(size_t)(n0 + nn) * K + k0 + kk] = (uint16_t)f32_to_bf16(tile[kk][nn]);
        }
    } else if (jb.kind == kPackColumnPair) {
        // out [K x 2N]: columns of W and W2 interleaved in blocks of 32 ([W 32 | W2 32] per 64)
        const uint16_t *w = (const uint16_t *)jb.src, *w2 = (const uint16_t *)jb.src2;
        uint16_t *out = (uint16_t *)jb.dst;
        const size_t total = (size_t)K * 2 * N;
        for (size_t x = (size_t)local * 4096 + tid; x < min(total, (size_t)(local + 1) * 4096); x += 256) {
            const int k = (int)(x / (2 * N)), nx = (int)(x % (2 * N));
            const uint16_t *src = (nx & 63) < 32 ? w : w2;
            out[x] = src[(size_t)k * N + (nx >> 6) * 32 + (nx & 31)];
        }
    } else if (jb.kind == kPackCopy) {
        // K x N 32-bit words
        const uint32_t *src = (const uint32_t *)jb.src;
        uint32_t *out = (uint32_t *)jb.dst;
        const size_t total = (size_t)K * N;
        for (size_t x = (size_t)local * 4096 + tid; x < min(total, (size_t)(local + 1) * 4096); x += 256) out[x] = src[x];
    } else {
        // pool keys: u[h][i] = W_k[i, 64h .. 64h + 63] . q_h / 8 (K = D, N = heads; src W_k, src2 the query)
        const uint16_t *wk = (const uint16_t *)jb.src, *q = (const uint16_t *)jb.src2;
        const int x = local * 256 + tid;
        if (x >= N * K) return;
        const int h = x / K, i = x % K;
        float sum = 0.f;
        for (int e = 0; e < 64; ++e) sum += bf16_to_f32(wk[(size_t)i * K + 64 * h + e]) * bf16_to_f32(q[64 * h + e]);
        ((float *)jb.dst)[x] = sum * 0.125f;
    }
}

}  // namespace

// (launchers follow)

hipError_t launch_attention_bwd(const AttnBwdArgs &a, hipStream_t stream) {
    if (a.ntiles == 0) return hipSuccess;
    k_attn_bwd_dq<<<a.ntiles * a.heads, 512, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_attn_bwd_dkv<<<a.ntiles * a.heads, 512, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t *gu, const uint16_t *da, uint16_t *dgu, uint16_t *a, int T, int F,
                             hipStream_t stream) {
    if (F % 32) return hipErrorInvalidValue;  // gate and up interleave in blocks of 32 features
    const size_t n = (size_t)T * (F / 8);
    if (!n) return hipSuccess;
    k_swiglu_bwd<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(gu, da, dgu, a, T, F);
    return hipGetLastError();
}

int rmsnorm_bwd_blocks(int T, int rows_per_block) { return (T + rows_per_block - 1) / rows_per_block; }

hipError_t launch_rmsnorm_bwd(const float *x, const float *gain, const float *dh, const float *dres, float *dx,
                              uint16_t *dxb, float *gpart, int rows_per_block, int T, int D, float eps,
                              hipStream_t stream) {
    const int blocks = rmsnorm_bwd_blocks(T, rows_per_block);
    if (!blocks) return hipSuccess;
#define UBE_RMSNORM_BWD(V, CM) \
    k_rmsnorm_bwd<V, CM><<<blocks, 256, 0, stream>>>(x, gain, dh, dres, dx, dxb, gpart, rows_per_block, T, D, eps)
    switch (D) {
        case 128: UBE_RMSNORM_BWD(2, 1); break;
        case 256: UBE_RMSNORM_BWD(4, 1); break;
        case 512: UBE_RMSNORM_BWD(4, 2); break;
        case 768: UBE_RMSNORM_BWD(4, 3); break;
        case 1024: UBE_RMSNORM_BWD(4, 4); break;
        case 384: UBE_RMSNORM_BWD(2, 3); break;
        case 640: UBE_RMSNORM_BWD(2, 5); break;
        case 896: UBE_RMSNORM_BWD(2, 7); break;
        default: return hipErrorInvalidValue;
    }
#undef UBE_RMSNORM_BWD
    return hipGetLastError();
}

hipError_t launch_sum_rows(const float *part, int blocks, int D, float *out, float *work, hipStream_t stream) {
    const int slices = (blocks + kColSlice - 1) / kColSlice;
    k_col_parts<<<dim3((D + 255) / 256, slices), 256, 0, stream>>>(part, blocks, D, work, 0, 0.f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_sum_rows<<<(D + 255) / 256, 256, 0, stream>>>(work, slices, D, out);
    return hipGetLastError();
}

void xty_split(int T, int M, int N, int *splits, int *chunk) {
    const bool wide = M % 256 == 0 && N % 256 == 0;
    const int tiles = wide ? (M / 256) * (N / 256) : (M / 128) * (N / 64);
    // as many ranges as fit one round of workgroups on the 256 CUs (one wide or two narrow workgroups per
    // CU): a partial second round would double the launch's time
    const int want = std::max(1, (wide ? 256 : 512) / tiles);
    const int cap = std::max(1, (T + 255) / 256);                  // at least 256 tokens per range
    int sp = std::max(1, std::min(want, cap));
    const int ch = ((T + sp - 1) / sp + 63) / 64 * 64;
    *chunk = std::max(ch, 64);
    *splits = std::max(1, (T + *chunk - 1) / *chunk);
}

hipError_t launch_xty(const uint16_t *x, int ldx, const uint16_t *y, int ldy, int T, int M, int N, float *partial,
                      float *out, float *out2, bool deinterleave, hipStream_t stream) {
    if (T <= 0 || M % 128 || N % 64) return hipErrorInvalidValue;
    int splits = 0, chunk = 0;
    xty_split(T, M, N, &splits, &chunk);
    if (M % 256 == 0 && N % 256 == 0)
        k_xty256<<<splits * (M / 256) * (N / 256), 512, 0, stream>>>(x, ldx, y, ldy, T, M, N, partial, chunk);
    else
        k_xty<<<splits * (M / 128) * (N / 64), 256, 0, stream>>>(x, ldx, y, ldy, T, M, N, partial, chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)M * N;
    k_xty_reduce<<<(unsigned)((n / 4 + 255) / 256), 256, 0, stream>>>(partial, splits, M, N, out, out2,
                                                                      deinterleave ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_embed_bwd(const float *dx, const uint32_t *tok_off, const uint32_t *tok, int V, int D, float *dE,
                            hipStream_t stream) {
    if (D > 1024 || D % 4) return hipErrorInvalidValue;
    k_embed_bwd<<<V, 512, 0, stream>>>(dx, tok_off, tok, D, dE);
    return hipGetLastError();
}

int pool_bwd_chunks(int count) { return std::max(1, std::min(16, 512 / std::max(count, 1))); }
int pool_bwd_token_ranges(int count) { return std::max(1, std::min(8, 256 / std::max(count, 1))); }

hipError_t launch_pool_bwd(const PoolBwdArgs &a, float *dz, float *pd, float *spa, float *zpart, float *dupart,
                           hipStream_t stream) {
    if (a.H > 16 || a.D > 1024 || a.D % 8) return hipErrorInvalidValue;
    hipError_t e;
    const int chunks = pool_bwd_chunks(a.count);
    if (a.count > 0) {
        k_pool_bwd_dz<<<dim3((a.H * a.D + 255) / 256, a.count), 256, 0, stream>>>(a, dz);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int tchunks = pool_bwd_token_ranges(a.count);
        if (a.D <= 512)
            k_pool_bwd_tokens<1><<<dim3(a.count, tchunks), 512, 0, stream>>>(a, dz, pd, spa, tchunks);
        else
            k_pool_bwd_tokens<2><<<dim3(a.count, tchunks), 512, 0, stream>>>(a, dz, pd, spa, tchunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_pool_bwd_cols<<<dim3((a.D + 255) / 256, a.count, chunks), 256, 0, stream>>>(a, dz, pd, spa, tchunks, zpart,
                                                                                        dupart, chunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_pool_bwd_item_sums<<<dim3((a.H * a.D + 255) / 256, a.count), 256, 0, stream>>>(a, zpart, dupart, chunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    float *du_tot = dz;  // dz is free once the columns pass ran
    k_pool_bwd_du<<<(a.H * a.D + 255) / 256, 256, 0, stream>>>(a, du_tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t n = (size_t)a.D * a.D + (size_t)a.D * 64;
    k_pool_bwd_weights<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a, du_tot);
    return hipGetLastError();
}

}  // namespace ube

namespace ube {

int adafactor_grids(AdaTensor *tab, int n, int *stats, int *cols, int *upd) {
    int g0 = 0, g1 = 0, g2 = 0;
    for (int i = 0; i < n; ++i) {
        AdaTensor &t = tab[i];
        const long long count = (long long)t.rows * (t.cols ? t.cols : 1);
        if (count <= 0 || count > 0x7fffffffLL) return -1;
        t.wg_stats = g0, t.wg_cols = g1, t.wg_upd = g2;
        g0 += t.cols ? (t.rows + kAdaSlice - 1) / kAdaSlice : (t.rows + 255) / 256;
        g1 += t.cols ? (t.cols + 255) / 256 : 0;
        g2 += (int)((count + kAdaChunk - 1) / kAdaChunk);
    }
    *stats = g0, *cols = g1, *upd = g2;
    return 0;
}

hipError_t launch_adafactor(const AdaTensor *tab, int n, int stats, int cols, int upd, const AdaStep &st,
                            hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    k_ada_stats<<<stats, 256, 0, stream>>>(tab, n, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (cols > 0) {
        k_ada_cols<<<cols, 256, 0, stream>>>(tab, n, st);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    k_ada_rms<<<upd, 256, 0, stream>>>(tab, n, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_ada_apply<<<upd, 256, 0, stream>>>(tab, n, st);
    return hipGetLastError();
}

int pack_workgroups(PackJob *jobs, int n) {
    int g = 0;
    for (int i = 0; i < n; ++i) {
        PackJob &j = jobs[i];
        j.first_wg = g;
        const size_t K = (size_t)j.K, N = (size_t)j.N;
        switch (j.kind) {
            case kPackTranspose: g += (int)(((N + 63) / 64) * ((K + 63) / 64)); break;
            case kPackTransposePair: g += (int)(((2 * N + 63) / 64) * ((K + 63) / 64)); break;
            case kPackColumnPair: g += (int)((K * 2 * N + 4095) / 4096); break;
            case kPackCopy: g += (int)((K * N + 4095) / 4096); break;
            default: g += (int)((K * N + 255) / 256); break;
        }
    }
    return g;
}

hipError_t launch_pack(const PackJob *jobs, int n, int workgroups, hipStream_t stream) {
    if (n <= 0 || workgroups <= 0) return hipSuccess;
    k_pack<<<workgroups, 256, 0, stream>>>(jobs, n);
    return hipGetLastError();
}

}  // namespace ube
