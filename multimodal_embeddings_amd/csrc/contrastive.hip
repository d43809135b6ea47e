// contrastive.hip -- gfx950 kernels of the Matryoshka sigmoid contrastive loss over pooled embeddings.
//
// What is computed: UForm overview page, "Matryoshka-Like Multi-Scale Embedders" (nested prefix widths,
// the SigLIP per-cell sigmoid loss with inverse temperature t and bias b); UForm for C training page,
// uform_contrastive_t (widths, temperature, bias, ambient weight), uform_negatives_t and
// uform_relations_view_t (edge precedence). Notation and the gradient split are in contrastive.h.
//
// Pipeline of one call (all on the caller's stream):
//   prefix norms -> named-edge corrections -> dense cells (scores, loss and gradient coefficients; the
//   coefficient blocks H_k land in HBM as bf16) -> row / column / scalar reductions in a fixed order ->
//   rows contraction (split over items) -> columns contraction (writes the gradient) -> named-edge
//   gradient terms.
// The dense cells are VALU-heavy (two transcendental ops and a transposed column reduction per cell and
// width); the two contractions are MFMA products whose A operand is read through the LDS transpose load
// (ds_read_b64_tr_b16), so neither operand needs a transposed copy in HBM.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "contrastive.h"
#include "device.h"

namespace ube {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Block of column d: the first width above it.
__device__ __forceinline__ int block_of(const ContrastiveArgs &a, int d) {
    int k = 0;
#pragma unroll
    for (int w = 0; w < kMaxWidths - 1; ++w)
        if (w < a.K - 1 && d >= a.widths[w]) k = w + 1;
    return k;
}

__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// ---------------------------------------------------------------------------------- LDS transpose load
//
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane i = 4a + b of a group receives element b of the
// 8 bytes read by lanes 4e + a of its group, e = 0..3, as its elements e. Reading row (kb + e) at
// column (c + 4a) in lane 4e + a therefore hands lane i the column c + i of rows kb .. kb + 3: four
// consecutive k of one column, the MFMA operand layout. Two such loads give the 8 k of a 32x32x16
// operand half.
//
// Tiles read this way are stored k-major (one row per k) in 16-byte chunks XOR-swizzled by the row:
// SW = 0 for 128-byte rows (chunk ^ 4 ((r / 2) % 2)), SW = 1 for 512-byte rows (chunk ^ 4 (r % 4)); the
// 32 lanes of a half-wave then cover 16 distinct 16-byte bank groups.
template <int SW>
__device__ __forceinline__ int tr_swz(int row) {
    return SW == 0 ? 4 * ((row >> 1) & 1) : 4 * (row & 3);
}

template <int PITCH, int SW>
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t *tile, int kb, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int col = c0 + 16 * (g & 1) + 4 * (i & 3);
    const int chunk = col >> 3, half = (col >> 2) & 1;
    const int r0 = kb + 8 * (g >> 1) + (i >> 2), r1 = r0 + 4;
    const uint8_t *p0 = tile + r0 * PITCH + ((chunk ^ tr_swz<SW>(r0)) << 4) + (half << 3);
    const uint8_t *p1 = tile + r1 * PITCH + ((chunk ^ tr_swz<SW>(r1)) << 4) + (half << 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

// Sum of 16 per-lane values over the 32 lanes of a half-wave (same lane / 32): each exchange keeps half
// of the values, so lane l ends with value r = 8 b4 + 4 b3 + 2 b2 + b1 (b = bits of l) summed over the
// half-wave; lanes l and l ^ 1 hold the same sum.
__device__ __forceinline__ float half_wave_reduce16(const float (&v)[16], int lane) {
    float c8[8], c4[4], c2[2];
    bool up = lane & 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) c8[j] = (up ? v[8 + j] : v[j]) + __shfl_xor(up ? v[j] : v[8 + j], 16, 64);
    up = lane & 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) c4[j] = (up ? c8[4 + j] : c8[j]) + __shfl_xor(up ? c8[j] : c8[4 + j], 8, 64);
    up = lane & 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) c2[j] = (up ? c4[2 + j] : c4[j]) + __shfl_xor(up ? c4[j] : c4[2 + j], 4, 64);
    up = lane & 2;
    float c1 = (up ? c2[1] : c2[0]) + __shfl_xor(up ? c2[0] : c2[1], 2, 64);
    return c1 + __shfl_xor(c1, 1, 64);
}

// ------------------------------------------------------------------------------------- prefix norms

// One wave per item: inv[w][i] = 1 / |e_i[:m_w]| (0 for a zero prefix), accumulated per block.
__global__ __launch_bounds__(256) void k_prefix_inv_norms(ContrastiveArgs a) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.n) return;
    const uint16_t *row = a.emb + (size_t)i * a.ld;
    const int mK = a.widths[a.K - 1];
    float bins[kMaxWidths];
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) bins[w] = 0.f;
    for (int c0 = lane; c0 * 8 < mK; c0 += 128) {
        u32x4 v[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = c0 + 64 * u;
            v[u] = c * 8 < mK ? *(const u32x4 *)(row + c * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            float ss = 0.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = bf16_to_f32(x[h] & 0xffff), hi = bf16_to_f32(x[h] >> 16);
                ss += lo * lo + hi * hi;
            }
            const int k = block_of(a, (c0 + 64 * u) * 8);
#pragma unroll
            for (int w = 0; w < kMaxWidths; ++w)
                if (w == k) bins[w] += ss;
        }
    }
    float cum = 0.f;
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        if (w < a.K) {
            cum += wave_sum(bins[w]);
            if (lane == 0) a.inv[(size_t)w * a.n + i] = cum > 0.f ? 1.0f / sqrtf(cum) : 0.f;
        }
    }
}

// ------------------------------------------------------------------------------------ named edges

// One wave per resolved edge: its exact prefix cosines, and what it changes against the dense pass
// (which scored the cell as an ambient negative when `dense`): delta gamma s, delta gamma, delta loss
// per width, and the delta coefficient of every block (suffix sums over widths).
__global__ __launch_bounds__(256) void k_contrastive_edges(ContrastiveArgs a) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= a.E) return;
    const ContrastiveEdge ed = a.edges[e];
    const int ia = a.r0 + ed.p, ij = ed.j;
    const uint16_t *ra = a.emb + (size_t)ia * a.ld, *rb = a.emb + (size_t)ij * a.ld;
    const int mK = a.widths[a.K - 1];
    float bins[kMaxWidths];
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) bins[w] = 0.f;
    for (int c = lane; c * 8 < mK; c += 64) {
        const u32x4 u = *(const u32x4 *)(ra + c * 8), v = *(const u32x4 *)(rb + c * 8);
        const uint32_t x[4] = {u.x, u.y, u.z, u.w}, y[4] = {v.x, v.y, v.z, v.w};
        float dot = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h)
            dot += bf16_to_f32(x[h] & 0xffff) * bf16_to_f32(y[h] & 0xffff) +
                   bf16_to_f32(x[h] >> 16) * bf16_to_f32(y[h] >> 16);
        const int k = block_of(a, c * 8);
#pragma unroll
        for (int w = 0; w < kMaxWidths; ++w)
            if (w == k) bins[w] += dot;
    }
    float out[4][kMaxWidths], dq[kMaxWidths];
    float dot = 0.f;
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        out[0][w] = out[1][w] = out[2][w] = out[3][w] = dq[w] = 0.f;
        if (w < a.K) {
            dot += wave_sum(bins[w]);
            const float ip = a.inv[(size_t)w * a.n + ia], iq = a.inv[(size_t)w * a.n + ij];
            const float s = dot * ip * iq, z = a.t * s + a.b;
            float g_d = 0.f, l_d = 0.f;
            if (a.dense) {
                g_d = a.c * a.wa / (1.f + expf(-z));
                l_d = a.wa * softplus(z);
            }
            float g_t = 0.f, l_t = 0.f;
            if (ed.y > 0) {
                g_t = -a.c * ed.w / (1.f + expf(z));  // w (sigma(z) - 1) = -w sigma(-z)
                l_t = ed.w * softplus(-z);
            } else if (ed.y < 0) {
                g_t = a.c * ed.w / (1.f + expf(-z));
                l_t = ed.w * softplus(z);
            }
            const float dg = g_t - g_d;
            out[0][w] = dg * s;
            out[1][w] = dg;
            out[2][w] = l_t - l_d;
            dq[w] = a.t * dg * ip * iq;
        }
    }
    float h = 0.f;
#pragma unroll
    for (int w = kMaxWidths - 1; w >= 0; --w) {
        if (w < a.K) {
            h += dq[w];
            out[3][w] = h;
        }
    }
    if (lane < 4 * kMaxWidths) {
        const int f = lane / kMaxWidths, w = lane % kMaxWidths;
        float v = 0.f;
#pragma unroll
        for (int ff = 0; ff < 4; ++ff)
#pragma unroll
            for (int ww = 0; ww < kMaxWidths; ++ww)
                if (ff == f && ww == w) v = out[ff][ww];
        if (w < a.K) a.edge_out[((size_t)e * 4 + f) * a.K + w] = v;
    }
}

// -------------------------------------------------------------------------------------- dense cells
//
// Workgroup tile: 128 items (j) x 128 anchors (p), 8 waves; wave (wj, wp) = (wave % 2, wave / 2) holds
// items 64 wj + [0, 64) (two MFMA tiles) of anchors 32 wp + [0, 32). MFMA A operand = item rows, B =
// anchor rows, so lane (l32, hh) holds anchor p = 32 wp + l32 and, in register 4 i + jj of tile tj, item
// 64 wj + 32 tj + 8 i + 4 hh + jj. The K loop runs over the columns in 64-wide stages; at the end of
// every width the running dot products are that width's prefix dots and the cells of the width are
// scored on the spot. The width's coefficients Q_w wait in registers (bf16) until the last width, when
// H_k = sum over w >= k of Q_w is formed and stored.

template <bool LOSS, bool GRAD, bool MASK>
__device__ __forceinline__ void score_width(const ContrastiveArgs &a, const f32x16 (&acc)[2], const float *sIJ,
                                            float ip, int p_item, int jbase, int lane, uint32_t (&q)[16],
                                            float &rowacc, float &gsum, float &lsum, float (&colres)[2]) {
    const int hh = lane >> 5;
    const float cpl = a.t * ip * kLog2e, bl = a.b * kLog2e;
    const float fq = a.t * a.c * a.wa * ip;
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        float col[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 ij4 = *(const f32x4 *)(sIJ + 32 * tj + 8 * i + 4 * hh);
            const float ijv[4] = {ij4.x, ij4.y, ij4.z, ij4.w};
            float qv[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float sp = acc[tj][4 * i + jj] * ijv[jj];
                const float z2 = fmaf(sp, cpl, bl);  // z log2(e)
                // u = 2^z2 (clamped: sigma is 1 to fp32 precision long before), sigma = u / (1 + u); the loss
                // reuses 1 + u: log2(1 + e^z) = log2(1 + u) (z2 itself past 24; u log2(e) below 2^-12)
                const float u = __builtin_amdgcn_exp2f(fminf(z2, 64.f));
                const float d = 1.f + u;
                float sig = u * __builtin_amdgcn_rcpf(d), l2 = 0.f;
                if constexpr (LOSS) {
                    l2 = u < 0x1p-12f ? u * kLog2e : __builtin_amdgcn_logf(d);
                    l2 = z2 > 24.f ? z2 : l2;
                }
                bool valid = true;
                if constexpr (MASK) {
                    const int j = jbase + 32 * tj + 8 * i + 4 * hh + jj;
                    valid = j < a.n && p_item >= 0 && j != p_item;
                    sig = valid ? sig : 0.f;
                }
                const float v = sig * (sp * ip);
                gsum += sig;
                rowacc += v;
                col[4 * i + jj] = v;
                if constexpr (LOSS) lsum += valid ? l2 : 0.f;
                if constexpr (GRAD) qv[jj] = sig * ijv[jj] * fq;
            }
            if constexpr (GRAD) {
                q[tj * 8 + 2 * i] = pack2(qv[0], qv[1]);
                q[tj * 8 + 2 * i + 1] = pack2(qv[2], qv[3]);
            }
        }
        if constexpr (GRAD) colres[tj] = half_wave_reduce16(col, lane);
    }
}

template <bool LOSS, bool GRAD>
__global__ __launch_bounds__(512, 1) void k_contrastive_cells(ContrastiveArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[4352];  // 2 stages x 256 rows x 8 chunks; H staging
    __shared__ __attribute__((aligned(16))) float sInvJ[kMaxWidths][128];
    __shared__ __attribute__((aligned(16))) float sInvP[kMaxWidths][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, wj = wave & 1, wp = wave >> 1;
    const int PT = a.R_pad >> 7;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int jt = logical / PT, pt = logical % PT;  // consecutive tiles share their items
    const int j0 = jt * 128, p0 = pt * 128;

    for (int idx = tid; idx < a.K * 128; idx += 512) {
        const int w = idx >> 7, r = idx & 127;
        sInvJ[w][r] = j0 + r < a.n ? a.inv[(size_t)w * a.n + j0 + r] : 0.f;
        sInvP[w][r] = p0 + r < a.R ? a.inv[(size_t)w * a.n + a.r0 + p0 + r] : 0.f;
    }
    // DMA round r (0..3): chunk slot 512 r + tid = tile row 64 r + tid / 8, LDS chunk tid % 8; rows
    // [0, 128) are items, [128, 256) anchors; rows past the end repeat the last one (their cells are masked)
    const int prow = tid >> 3, pch = tid & 7;
    const uint16_t *src[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 64 * r + prow;
        const int item = row < 128 ? min(j0 + row, a.n - 1) : a.r0 + min(p0 + row - 128, a.R - 1);
        src[r] = a.emb + (size_t)item * a.ld + swz(row, pch) * 8;
    }
    auto issue = [&](int k0, int buf) {
#pragma unroll
        for (int r = 0; r < 4; ++r) lds_dma16(src[r] + k0, smem + buf * 2048 + r * 512 + wave * 64);
    };
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    auto compute = [&](int buf) {
        const u32x4 *sJ = smem + buf * 2048, *sP = sJ + 128 * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 2 * ks + hh;
            const int rj = 64 * wj + l32, rp = 32 * wp + l32;
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, sJ[rj * 8 + swz(rj, ch)]);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, sJ[(rj + 32) * 8 + swz(rj + 32, ch)]);
            const bf16x8 bp = __builtin_bit_cast(bf16x8, sP[rp * 8 + swz(rp, ch)]);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bp, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bp, acc[1], 0, 0, 0);
        }
    };

    uint32_t q[kMaxWidths][16];
    float rowacc[kMaxWidths], gsum[kMaxWidths], lsum[kMaxWidths], colres[kMaxWidths][2];
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        rowacc[w] = gsum[w] = lsum[w] = colres[w][0] = colres[w][1] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) q[w][r] = 0u;
    }
    const int p_local = 32 * wp + l32;
    const int p_item = p0 + p_local < a.R ? a.r0 + p0 + p_local : -1;
    const int ja = a.r0 + p0, jb = a.r0 + min(p0 + 128, a.R);  // anchor items of the tile
    const bool interior = j0 + 128 <= a.n && p0 + 128 <= a.R && (jb <= j0 || j0 + 128 <= ja);
    const int jbase = j0 + 64 * wj;
    const int nk = a.widths[a.K - 1] >> 6;

    issue(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            issue((kt + 1) * 64, buf ^ 1);
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        lds_barrier();
        compute(buf);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        const int kend = (kt + 1) * 64;
#pragma unroll
        for (int w = 0; w < kMaxWidths; ++w) {
            if (w < a.K && a.widths[w] == kend) {
                const float ip = sInvP[w][p_local];
                if (interior)
                    score_width<LOSS, GRAD, false>(a, acc, &sInvJ[w][64 * wj], ip, p_item, jbase, lane, q[w],
                                                   rowacc[w], gsum[w], lsum[w], colres[w]);
                else
                    score_width<LOSS, GRAD, true>(a, acc, &sInvJ[w][64 * wj], ip, p_item, jbase, lane, q[w],
                                                  rowacc[w], gsum[w], lsum[w], colres[w]);
            }
        }
    }

    if constexpr (GRAD) {
        // H_k = Q_k + H_{k+1}, widest first; each block goes through LDS (rows of 128 items, 272-byte pitch)
        // so that every global store writes 16 bytes of a contiguous 256-byte row segment
        constexpr int kPitch = 272;
        uint8_t *stg = (uint8_t *)smem;
        const size_t hstride = (size_t)a.R_pad * a.n_pad;
        float h[2][4][4];
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) h[tj][i][jj] = 0.f;
#pragma unroll
        for (int w = kMaxWidths - 1; w >= 0; --w) {
            if (w < a.K) {
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t x0 = q[w][tj * 8 + 2 * i], x1 = q[w][tj * 8 + 2 * i + 1];
                        h[tj][i][0] += bf16_to_f32(x0 & 0xffff);
                        h[tj][i][1] += bf16_to_f32(x0 >> 16);
                        h[tj][i][2] += bf16_to_f32(x1 & 0xffff);
                        h[tj][i][3] += bf16_to_f32(x1 >> 16);
                        *(u32x2 *)(stg + p_local * kPitch + (64 * wj + 32 * tj + 8 * i + 4 * hh) * 2) =
                            u32x2{pack2(h[tj][i][0], h[tj][i][1]), pack2(h[tj][i][2], h[tj][i][3])};
                    }
                __syncthreads();
                uint16_t *hw = a.H + (size_t)w * hstride + (size_t)p0 * a.n_pad + j0;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int c = tid + 512 * x, row = c >> 4, ch = c & 15;
                    *(u32x4 *)(hw + (size_t)row * a.n_pad + ch * 8) = *(const u32x4 *)(stg + row * kPitch + ch * 16);
                }
                __syncthreads();
            }
        }
    }

    // fixed-order reductions through LDS (the operand stages are free after the loop's last barrier)
    float *sRow = (float *)smem;                  // [K][2 wj][128 p]
    float *sCol = sRow + kMaxWidths * 256;        // [K][4 wp][128 j]
    float *sWg = sCol + kMaxWidths * 512;         // [K][8 waves][2]
    const int ib = 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1), jb2 = 2 * ((lane >> 2) & 1) + ((lane >> 1) & 1);
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        if (w < a.K) {
            const float r = rowacc[w] + __shfl_xor(rowacc[w], 32, 64);
            if (hh == 0) sRow[(w * 2 + wj) * 128 + p_local] = r;
            if (GRAD && (lane & 1) == 0) {
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    sCol[(w * 4 + wp) * 128 + 64 * wj + 32 * tj + 8 * ib + 4 * hh + jb2] = colres[w][tj];
            }
            const float g = wave_sum(gsum[w]);
            const float l = LOSS ? wave_sum(lsum[w]) : 0.f;
            if (lane == 0) {
                sWg[(w * 8 + wave) * 2] = g;
                sWg[(w * 8 + wave) * 2 + 1] = l;
            }
        }
    }
    __syncthreads();
    const float cwa = a.c * a.wa;
    for (int idx = tid; idx < a.K * 128; idx += 512) {
        const int w = idx >> 7, r = idx & 127;
        a.rowpart[((size_t)jt * a.K + w) * a.R_pad + p0 + r] = cwa * (sRow[(w * 2) * 128 + r] + sRow[(w * 2 + 1) * 128 + r]);
        if constexpr (GRAD) {
            const float *c = sCol + w * 512 + r;
            a.colpart[((size_t)pt * a.K + w) * a.n_pad + j0 + r] = cwa * (((c[0] + c[128]) + c[256]) + c[384]);
        }
    }
    if (tid < a.K) {
        float g = 0.f, l = 0.f;
        for (int v = 0; v < 8; ++v) {
            g += sWg[(tid * 8 + v) * 2];
            l += sWg[(tid * 8 + v) * 2 + 1];
        }
        a.wgpart[((size_t)logical * a.K + tid) * 2] = cwa * g;
        a.wgpart[((size_t)logical * a.K + tid) * 2 + 1] = a.wa * kLn2 * l;
    }
}

// -------------------------------------------------------------------------------------- reductions

// Per anchor and width: rho from the item-tile partials plus the anchor's edges (in order), and the raw
// sum of gamma s (the anchor's share of d loss / d t). Workgroup = 64 anchors x one width; its 8 waves
// split the item tiles into eight fixed ranges.
__global__ __launch_bounds__(512) void k_contrastive_rows(ContrastiveArgs a) {
    __shared__ float part[8][64];
    const int tid = threadIdx.x, pl = tid & 63, sl = tid >> 6;
    const int p = blockIdx.x * 64 + pl, w = blockIdx.y;
    const int JT = a.n_pad >> 7;
    const int lo = (int)((long)JT * sl / 8), hi = (int)((long)JT * (sl + 1) / 8);
    float s = 0.f;
    if (a.dense) {
        const float *src = a.rowpart + (size_t)w * a.R_pad + p;
        const size_t step = (size_t)a.K * a.R_pad;
        int jt = lo;
        float s1 = 0.f, s2 = 0.f, s3 = 0.f;
        for (; jt + 4 <= hi; jt += 4) {
            s += src[(size_t)jt * step];
            s1 += src[(size_t)(jt + 1) * step];
            s2 += src[(size_t)(jt + 2) * step];
            s3 += src[(size_t)(jt + 3) * step];
        }
        for (; jt < hi; ++jt) s += src[(size_t)jt * step];
        s = (s + s1) + (s2 + s3);
    }
    part[sl][pl] = s;
    __syncthreads();
    if (sl != 0) return;
    float tot = 0.f, rho = 0.f;
    if (p < a.R) {
        for (int v = 0; v < 8; ++v) tot += part[v][pl];
        if (a.E)
            for (uint32_t e = a.row_edges[p]; e < a.row_edges[p + 1]; ++e) tot += a.edge_out[((size_t)e * 4) * a.K + w];
        const float ip = a.inv[(size_t)w * a.n + a.r0 + p];
        rho = a.t * ip * ip * tot;
    }
    a.rho[(size_t)w * a.R_pad + p] = rho;
    a.rsum[(size_t)w * a.R_pad + p] = tot;
}

// Block coefficient of rho for anchor p and column block k: the sum over widths w >= k.
__device__ __forceinline__ float rho_block(const ContrastiveArgs &a, int k, int p) {
    float h = 0.f;
#pragma unroll
    for (int w = kMaxWidths - 1; w >= 0; --w)
        if (w < a.K && w >= k) h += a.rho[(size_t)w * a.R_pad + p];
    return h;
}

// Per item: kappa of every width from the anchor-tile partials plus the item's incoming edges.
__global__ __launch_bounds__(256) void k_contrastive_cols(ContrastiveArgs a) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= a.n_pad) return;
    const int PT = a.R_pad >> 7;
    float kap[kMaxWidths];
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        kap[w] = 0.f;
        if (w < a.K && j < a.n) {
            float s = 0.f;
            if (a.dense)
                for (int pt = 0; pt < PT; ++pt) s += a.colpart[((size_t)pt * a.K + w) * a.n_pad + j];
            if (a.E)
                for (uint32_t x = a.col_offsets[j]; x < a.col_offsets[j + 1]; ++x)
                    s += a.edge_out[((size_t)a.col_edges[x] * 4) * a.K + w];
            const float iq = a.inv[(size_t)w * a.n + j];
            kap[w] = a.t * iq * iq * s;
        }
    }
    float h = 0.f;
#pragma unroll
    for (int w = kMaxWidths - 1; w >= 0; --w) {
        if (w < a.K) {
            h += kap[w];
            a.kappa_blk[(size_t)w * a.n_pad + j] = h;
        }
    }
}

// The scalars: width losses, d loss / d t, d loss / d b; every sum in a fixed order (a fixed share per
// thread, then wave sums, then the 16 waves in order).
__global__ __launch_bounds__(1024) void k_contrastive_scalars(ContrastiveArgs a) {
    __shared__ float red[16][2 * kMaxWidths + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tiles = a.dense ? (a.R_pad >> 7) * (a.n_pad >> 7) : 0;
    float g[kMaxWidths], l[kMaxWidths], dt = 0.f;
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) g[w] = l[w] = 0.f;
    for (int x = tid; x < tiles; x += 1024) {
#pragma unroll
        for (int w = 0; w < kMaxWidths; ++w) {
            if (w < a.K) {
                const float2 v = *(const float2 *)(a.wgpart + ((size_t)x * a.K + w) * 2);
                g[w] += v.x;
                l[w] += v.y;
            }
        }
    }
    for (int e = tid; e < a.E; e += 1024) {
#pragma unroll
        for (int w = 0; w < kMaxWidths; ++w) {
            if (w < a.K) {
                g[w] += a.edge_out[((size_t)e * 4 + 1) * a.K + w];
                l[w] += a.edge_out[((size_t)e * 4 + 2) * a.K + w];
            }
        }
    }
    for (int idx = tid; idx < a.K * a.R_pad; idx += 1024)
        if (idx % a.R_pad < a.R) dt += a.rsum[idx];
#pragma unroll
    for (int w = 0; w < kMaxWidths; ++w) {
        if (w < a.K) {
            const float gs = wave_sum(g[w]), ls = wave_sum(l[w]);
            if (lane == 0) {
                red[wave][2 * w] = gs;
                red[wave][2 * w + 1] = ls;
            }
        }
    }
    dt = wave_sum(dt);
    if (lane == 0) red[wave][2 * kMaxWidths] = dt;
    __syncthreads();
    if (tid != 0) return;
    float db = 0.f, loss = 0.f, dts = 0.f;
    for (int v = 0; v < 16; ++v) dts += red[v][2 * kMaxWidths];
    for (int w = 0; w < a.K; ++w) {
        float gw = 0.f, lw = 0.f;
        for (int v = 0; v < 16; ++v) {
            gw += red[v][2 * w];
            lw += red[v][2 * w + 1];
        }
        lw /= (float)a.R;
        db += gw;
        loss += lw;
        a.scalars[3 + w] = a.want_loss ? lw : __builtin_nanf("");
    }
    a.scalars[0] = a.want_loss ? loss / (float)a.K : __builtin_nanf("");
    a.scalars[1] = dts;
    a.scalars[2] = db;
}

// ------------------------------------------------------------------------------------ contractions
//
// Both contractions compute 64 columns (d, one block) x 256 cells per workgroup (4 waves, 64 cells
// each, 2 x 2 MFMA tiles), A operand = embedding columns read k-major through the transpose load, so
// that lane (l32, hh) ends with 4 consecutive columns of one cell row in each register group: 16-byte
// stores of the fp32 gradient.

constexpr int kGradStage = 2560;  // 16-byte chunks per stage: 2048 coefficients + 512 embedding columns

// rows: partial[s][p][d] = sum over items j of the split of H_k(p, j) e_j[d]
__global__ __launch_bounds__(256, 2) void k_contrastive_grad_rows(ContrastiveArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[2 * kGradStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int DT = a.widths[a.K - 1] >> 6, PT = a.R_pad >> 8;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int dtile = logical % DT, rest = logical / DT, pt = rest % PT, s = rest / PT;
    const int d0 = dtile * 64, p0 = pt * 256;
    const int k = block_of(a, d0);
    const uint16_t *Hk = a.H + (size_t)k * a.R_pad * a.n_pad;
    const int jbeg = s * a.chunk, jend = min(a.n_pad, jbeg + a.chunk);
    f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
    // coefficient rows (anchors, 128 bytes = 64 items per stage): round r (0..7) moves slot 256 r + tid
    const int hrow = tid >> 3, hch = tid & 7;
    auto issue = [&](int jb, int buf) {
        u32x4 *st = smem + buf * kGradStage;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = 32 * r + hrow;
            lds_dma16(Hk + (size_t)(p0 + row) * a.n_pad + jb + swz(row, hch) * 8, st + r * 256 + wave * 64);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 32 * r + hrow;  // item jb + row, 64 columns from d0
            const int item = min(jb + row, a.n - 1);
            lds_dma16(a.emb + (size_t)item * a.ld + d0 + ((hch ^ tr_swz<0>(row)) << 3), st + 2048 + r * 256 + wave * 64);
        }
    };
    auto compute = [&](int buf) {
        const u32x4 *sH = smem + buf * kGradStage;
        const uint8_t *sE = (const uint8_t *)(sH + 2048);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 A[2], B[2];
#pragma unroll
            for (int td = 0; td < 2; ++td) A[td] = tr_frag<128, 0>(sE, 16 * ks, 32 * td, lane);
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const int row = 64 * wave + 32 * tp + l32, ch = 2 * ks + hh;
                B[tp] = __builtin_bit_cast(bf16x8, sH[row * 8 + swz(row, ch)]);
            }
#pragma unroll
            for (int td = 0; td < 2; ++td)
#pragma unroll
                for (int tp = 0; tp < 2; ++tp)
                    acc[td][tp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[td], B[tp], acc[td][tp], 0, 0, 0);
        }
    };
    const int nk = jend > jbeg ? (jend - jbeg) >> 6 : 0;
    if (nk) issue(jbeg, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            issue(jbeg + (kt + 1) * 64, buf ^ 1);
            asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        lds_barrier();
        compute(buf);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
    }
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        const int p = p0 + 64 * wave + 32 * tp + l32;
        float *out = a.rows_partial + ((size_t)s * a.R_pad + p) * a.D + d0 + 4 * hh;
#pragma unroll
        for (int td = 0; td < 2; ++td)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(f32x4 *)(out + 32 * td + 8 * i) =
                    f32x4{acc[td][tp][4 * i], acc[td][tp][4 * i + 1], acc[td][tp][4 * i + 2], acc[td][tp][4 * i + 3]};
    }
}

// rows_final[p][d] = sum over splits of the partials - (block coefficient of rho) e_p[d]
__global__ __launch_bounds__(256) void k_contrastive_rows_finish(ContrastiveArgs a) {
    const int D4 = a.D >> 2;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.R * D4) return;
    const int p = (int)(idx / D4), d = (int)(idx % D4) * 4;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    if (d < a.widths[a.K - 1]) {
        for (int sp = 0; sp < a.splits; ++sp) s += *(const f32x4 *)(a.rows_partial + ((size_t)sp * a.R_pad + p) * a.D + d);
        const float rho = rho_block(a, block_of(a, d), p);
        const u32x2 e = *(const u32x2 *)(a.emb + (size_t)(a.r0 + p) * a.ld + d);
        s.x -= rho * bf16_to_f32(e.x & 0xffff);
        s.y -= rho * bf16_to_f32(e.x >> 16);
        s.z -= rho * bf16_to_f32(e.y & 0xffff);
        s.w -= rho * bf16_to_f32(e.y >> 16);
    }
    *(f32x4 *)(a.rows_final + (size_t)p * a.D + d) = s;
}

// columns: grad[j][d] = sum over anchors p of H_k(p, j) e_p[d] - (block coefficient of kappa) e_j[d]
//          + rows_final[j - r0][d] when item j is an anchor; columns past the widest width are 0.
__global__ __launch_bounds__(256, 2) void k_contrastive_grad_cols(ContrastiveArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[2 * kGradStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int DTall = a.D >> 6;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int jt = logical / DTall, dtile = logical % DTall;  // consecutive tiles share their coefficients
    const int j0 = jt * 256, d0 = dtile * 64;
    if (d0 >= a.widths[a.K - 1]) {
        for (int x = tid; x < 256 * 16; x += 256) {
            const int j = j0 + (x >> 4), d = d0 + (x & 15) * 4;
            if (j < a.n) *(f32x4 *)(a.grad + (size_t)j * a.gld + d) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }
    const int k = block_of(a, d0);
    const uint16_t *Hk = a.H + (size_t)k * a.R_pad * a.n_pad;
    f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
    // coefficient rows (64 anchors x 256 items, 512 bytes each): round r (0..7) moves slot 256 r + tid
    const int hrow = tid >> 5, hch = tid & 31;
    const int erow = tid >> 3, ech = tid & 7;
    auto issue = [&](int pb, int buf) {
        u32x4 *st = smem + buf * kGradStage;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = 8 * r + hrow;
            lds_dma16(Hk + (size_t)(pb + row) * a.n_pad + j0 + ((hch ^ tr_swz<1>(row)) << 3), st + r * 256 + wave * 64);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 32 * r + erow;
            const int item = a.r0 + min(pb + row, a.R - 1);
            lds_dma16(a.emb + (size_t)item * a.ld + d0 + ((ech ^ tr_swz<0>(row)) << 3), st + 2048 + r * 256 + wave * 64);
        }
    };
    auto compute = [&](int buf) {
        const uint8_t *sH = (const uint8_t *)(smem + buf * kGradStage);
        const uint8_t *sE = sH + 2048 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 A[2], B[2];
#pragma unroll
            for (int td = 0; td < 2; ++td) A[td] = tr_frag<128, 0>(sE, 16 * ks, 32 * td, lane);
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) B[tj] = tr_frag<512, 1>(sH, 16 * ks, 64 * wave + 32 * tj, lane);
#pragma unroll
            for (int td = 0; td < 2; ++td)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    acc[td][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[td], B[tj], acc[td][tj], 0, 0, 0);
        }
    };
    const int nk = a.R_pad >> 6;
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            issue((kt + 1) * 64, buf ^ 1);
            asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        lds_barrier();
        compute(buf);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
    }
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        const int j = j0 + 64 * wave + 32 * tj + l32;
        if (j >= a.n) continue;
        const float kap = a.kappa_blk[(size_t)k * a.n_pad + j];
        const bool anchor = j >= a.r0 && j < a.r0 + a.R;
        const uint16_t *erow_p = a.emb + (size_t)j * a.ld;
#pragma unroll
        for (int td = 0; td < 2; ++td)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = d0 + 32 * td + 8 * i + 4 * hh;
                const u32x2 e = *(const u32x2 *)(erow_p + d);
                f32x4 o = f32x4{acc[td][tj][4 * i], acc[td][tj][4 * i + 1], acc[td][tj][4 * i + 2], acc[td][tj][4 * i + 3]};
                o.x -= kap * bf16_to_f32(e.x & 0xffff);
                o.y -= kap * bf16_to_f32(e.x >> 16);
                o.z -= kap * bf16_to_f32(e.y & 0xffff);
                o.w -= kap * bf16_to_f32(e.y >> 16);
                if (anchor) o += *(const f32x4 *)(a.rows_final + (size_t)(j - a.r0) * a.D + d);
                *(f32x4 *)(a.grad + (size_t)j * a.gld + d) = o;
            }
    }
}

// No dense cells (named negatives): grad[j][d] = -(kappa + rho) e_j[d] per block, 0 past the widest width.
__global__ __launch_bounds__(256) void k_contrastive_diag(ContrastiveArgs a) {
    const int D4 = a.D >> 2;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.n * D4) return;
    const int j = (int)(idx / D4), d = (int)(idx % D4) * 4;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    if (d < a.widths[a.K - 1]) {
        const int k = block_of(a, d);
        float c = a.kappa_blk[(size_t)k * a.n_pad + j];
        if (j >= a.r0 && j < a.r0 + a.R) c += rho_block(a, k, j - a.r0);
        const u32x2 e = *(const u32x2 *)(a.emb + (size_t)j * a.ld + d);
        o = f32x4{-c * bf16_to_f32(e.x & 0xffff), -c * bf16_to_f32(e.x >> 16), -c * bf16_to_f32(e.y & 0xffff),
                  -c * bf16_to_f32(e.y >> 16)};
    }
    *(f32x4 *)(a.grad + (size_t)j * a.gld + d) = o;
}

// Named-edge terms of the gradient: one wave per item that an edge touches; its outgoing edges (as an
// anchor) and incoming ones (as a candidate) in a fixed order, added onto the dense gradient row.
__global__ __launch_bounds__(64) void k_contrastive_sparse(ContrastiveArgs a) {
    const int lane = threadIdx.x;
    const int i = (int)a.touched[blockIdx.x];
    const bool anchor = i >= a.r0 && i < a.r0 + a.R;
    const uint32_t rb = anchor ? a.row_edges[i - a.r0] : 0u, re = anchor ? a.row_edges[i - a.r0 + 1] : 0u;
    const uint32_t cb = a.col_offsets[i], ce = a.col_offsets[i + 1];
    const int mK = a.widths[a.K - 1];
    for (int c = lane; c * 8 < mK; c += 64) {
        const int d = c * 8, k = block_of(a, d);
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto add = [&](uint32_t e, int item) {
            const float h = a.edge_out[((size_t)e * 4 + 3) * a.K + k];
            const u32x4 v = *(const u32x4 *)(a.emb + (size_t)item * a.ld + d);
            const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[2 * q] += h * bf16_to_f32(x[q] & 0xffff);
                s[2 * q + 1] += h * bf16_to_f32(x[q] >> 16);
            }
        };
        for (uint32_t e = rb; e < re; ++e) add(e, a.edges[e].j);
        for (uint32_t x = cb; x < ce; ++x) {
            const uint32_t e = a.col_edges[x];
            add(e, a.r0 + a.edges[e].p);
        }
        float *g = a.grad + (size_t)i * a.gld + d;
        f32x4 g0 = *(f32x4 *)g, g1 = *(f32x4 *)(g + 4);
        g0 += f32x4{s[0], s[1], s[2], s[3]};
        g1 += f32x4{s[4], s[5], s[6], s[7]};
        *(f32x4 *)g = g0;
        *(f32x4 *)(g + 4) = g1;
    }
}

}  // namespace

hipError_t launch_prefix_inv_norms(const ContrastiveArgs &a, hipStream_t stream) {
    if (a.n <= 0) return hipSuccess;
    k_prefix_inv_norms<<<(a.n + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_contrastive_edges(const ContrastiveArgs &a, hipStream_t stream) {
    if (a.E <= 0) return hipSuccess;
    k_contrastive_edges<<<(a.E + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_contrastive_cells(const ContrastiveArgs &a, bool grad, hipStream_t stream) {
    if (!a.dense) return hipSuccess;
    const int tiles = (a.R_pad >> 7) * (a.n_pad >> 7);
    if (a.want_loss && grad) k_contrastive_cells<true, true><<<tiles, 512, 0, stream>>>(a);
    else if (a.want_loss) k_contrastive_cells<true, false><<<tiles, 512, 0, stream>>>(a);
    else if (grad) k_contrastive_cells<false, true><<<tiles, 512, 0, stream>>>(a);
    else k_contrastive_cells<false, false><<<tiles, 512, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_contrastive_reduce(const ContrastiveArgs &a, bool grad, hipStream_t stream) {
    k_contrastive_rows<<<dim3(a.R_pad / 64, a.K), 512, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (grad) {
        k_contrastive_cols<<<a.n_pad / 256, 256, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    k_contrastive_scalars<<<1, 1024, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_contrastive_grad_rows(const ContrastiveArgs &a, hipStream_t stream) {
    if (!a.dense) return hipSuccess;
    const int DT = a.widths[a.K - 1] >> 6;
    k_contrastive_grad_rows<<<a.splits * (a.R_pad >> 8) * DT, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n4 = (size_t)a.R * (a.D >> 2);
    k_contrastive_rows_finish<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_contrastive_grad_cols(const ContrastiveArgs &a, hipStream_t stream) {
    if (a.dense) {
        k_contrastive_grad_cols<<<(a.n_pad >> 8) * (a.D >> 6), 256, 0, stream>>>(a);
    } else {
        const size_t n4 = (size_t)a.n * (a.D >> 2);
        k_contrastive_diag<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_contrastive_sparse(const ContrastiveArgs &a, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    k_contrastive_sparse<<<a.T, 64, 0, stream>>>(a);
    return hipGetLastError();
}

// No anchors: the loss and every gradient are zero (the width losses too, or NaN when not asked for).
__global__ void k_contrastive_empty(ContrastiveArgs a) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < 3 + (size_t)a.K) a.scalars[idx] = (a.want_loss || idx == 1 || idx == 2) ? 0.f : __builtin_nanf("");
    if (a.grad) {
        const size_t D4 = a.D >> 2;
        for (size_t x = idx; x < (size_t)a.n * D4; x += (size_t)gridDim.x * 256)
            *(f32x4 *)(a.grad + (x / D4) * a.gld + (x % D4) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

hipError_t launch_contrastive_empty(const ContrastiveArgs &a, hipStream_t stream) {
    k_contrastive_empty<<<256, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ube
