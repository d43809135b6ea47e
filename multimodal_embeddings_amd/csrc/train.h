// train.h -- launch interface of the gfx950 kernels of the encoder's backward pass and the Adafactor
// update (internal to libube).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ube {

// Attention backward for one head width of 64: rows of q, k (after the rotary), dO and O, feature-major v;
// the softmax
// log2 denominators (lse, head-major, base-2 units of log2(e) q.k / 8); delta = rowsum(dO * O) per query
// and head is formed by the dQ kernel into `delta`; tiles as the forward's (item, first token) list of
// 256-token tiles.
struct AttnBwdArgs {
    const uint16_t *q, *k;
    int ldqk;
    const uint16_t *vt;  // v feature-major [D x ldvt] (as the forward's QKV product writes it)
    int ldvt;
    const uint16_t *dout;
    int lddo;
    const float *lse;
    float *delta;  // written by the dQ kernel: rowsum(dO * O) per (head, query), read by the dK/dV kernel
    int ldl;
    const uint16_t *o;  // attention output rows (for delta)
    int ldo;
    uint16_t *dq, *dk, *dv;  // rows of ldd elements (e.g. the three parts of one [T x 3D] buffer)
    int ldd;
    const int *cu;
    const int2 *tiles;
    int ntiles;
    int heads;
    // 1-axis rotary (positions pos[t * 4], table rope[pos * 32 + pair] of (cos, sin)): when set, dq and dk
    // are written through the transposed rotation, i.e. with respect to q and k before the rotary
    const int16_t *pos;
    const float2 *rope;
};
hipError_t launch_attention_bwd(const AttnBwdArgs &a, hipStream_t stream);
// SwiGLU backward: gu [T x 2F] interleaved in blocks of 32 (gate | up), da [T x F] -> dgu (same interleave)
// and a = SiLU(g) u [T x F]
hipError_t launch_swiglu_bwd(const uint16_t *gu, const uint16_t *da, uint16_t *dgu, uint16_t *a, int T, int F,
                             hipStream_t stream);
// RMSNorm backward with residual (D a multiple of 128, at most 1024): dx = dres + d/dx <rmsnorm(x) * g, dh>; dxb = bf16(dx) (optional);
// gain partials gpart[block][D] = sum over the block's rows of dh * x / rms (rows_per_block rows each)
hipError_t launch_rmsnorm_bwd(const float *x, const float *gain, const float *dh, const float *dres, float *dx,
                              uint16_t *dxb, float *gpart, int rows_per_block, int T, int D, float eps,
                              hipStream_t stream);
int rmsnorm_bwd_blocks(int T, int rows_per_block);
// out[m][n] = sum over t of X[t][m] Y[t][n] (bf16 operands, fp32 partials per range of t, then reduced in
// range order); M % 128 == 0, N % 64 == 0. With `deinterleave`, n runs over [gate 32 | up 32] blocks and
// out receives the gate columns, out2 the up columns ([M x N/2] each). xty_split gives the ranges the
// launch uses: `partial` holds splits * M * N floats.
void xty_split(int T, int M, int N, int *splits, int *chunk);
hipError_t launch_xty(const uint16_t *x, int ldx, const uint16_t *y, int ldy, int T, int M, int N, float *partial,
                      float *out, float *out2, bool deinterleave, hipStream_t stream);
// columns sums of fixed blocks: out[d] = sum over b < blocks of part[b][d]
// work: at least ceil(blocks / 32) * D floats
hipError_t launch_sum_rows(const float *part, int blocks, int D, float *out, float *work, hipStream_t stream);
// Embedding gradient: dE[v] = sum over tokens of byte v (host-sorted lists) of dx[t]
hipError_t launch_embed_bwd(const float *dx, const uint32_t *tok_off, const uint32_t *tok, int V, int D, float *dE,
                            hipStream_t stream);
// Pool backward per item (see train.hip); writes dxf [T x D] fp32, per-item z and du for the weight
// gradients, then the gradients of W_v, W_k and the pool query.
struct PoolBwdArgs {
    const uint16_t *xf;   // [T x D] final-norm rows
    const float *s;       // [T x H] pool scores xf . u_h
    const int *cu;
    int count, D, H;
    const float *u;       // [H x D]
    const uint16_t *wv;   // [D x D] canonical
    const uint16_t *wk;   // [D x D] canonical
    const uint16_t *query;  // [D]
    const float *dpooled; // [count x D]
    float *dxf;           // [T x D]
    float *z, *du;        // [count x H x D] work
    float *dwv, *dwk, *dquery;  // [D x D], [D x D], [D]
};
// Work buffers: dz [count x H x D], pd [T x H x 2], spa [count x ranges x H] with ranges =
// pool_bwd_token_ranges(count), zpart and dupart [count x chunks x H x D] each with chunks =
// pool_bwd_chunks(count). D % 8 == 0, D <= 1024, H <= 16.
int pool_bwd_chunks(int count);
int pool_bwd_token_ranges(int count);
hipError_t launch_pool_bwd(const PoolBwdArgs &a, float *dz, float *pd, float *spa, float *zpart, float *dupart,
                           hipStream_t stream);

// Adafactor over every tensor of a model in four launches. One table entry per tensor (device memory,
// built once): gradient g fp32; master bf16 (w16) or fp32 (w32); state r [rows], c [cols] (matrices) or
// v [rows] (vectors), m [rows x cols]; work: col_parts [ceil(rows / kAdaSlice) x cols], rms_parts
// [ceil(count / kAdaChunk)], mean_r [1]. adafactor_grids fills the wg_* fields (host copy of the table)
// and the three grid sizes; -1 for an empty tensor or one of 2^31 elements or more.
constexpr int kAdaSlice = 32;
constexpr int kAdaChunk = 4096;
struct AdaTensor {
    const float *g;
    uint16_t *w16;
    float *w32;
    float *r, *c, *v, *m;
    float *col_parts, *rms_parts, *mean_r;
    int rows, cols;  // cols == 0: a vector of `rows`
    int wg_stats, wg_cols, wg_upd;
};
struct AdaStep {
    float lr, beta1, beta2, eps1, clip, bias_correction;
};
int adafactor_grids(AdaTensor *table, int n, int *stats, int *cols, int *upd);
hipError_t launch_adafactor(const AdaTensor *table, int n, int stats, int cols, int upd, const AdaStep &step,
                            hipStream_t stream);

// The derived copies of the masters in one launch, from a device table of jobs (pack_workgroups fills
// first_wg on the host copy and returns the grid size):
//   kPackTranspose:     dst[n][k] = bf16(src[k][n] * (gain ? gain[k] : 1)), src [K x N] bf16
//   kPackTransposePair: the same over the pair (src, src2) [K x N] each, dst rows running over
//                       [src 32 | src2 32] column blocks ([2N x K])
//   kPackColumnPair:    dst [K x 2N], the columns of src and src2 interleaved in blocks of 32
//   kPackCopy:          K x N 32-bit words
//   kPackPoolKeys:      dst[h][i] = src[i, 64h .. 64h + 63] . src2[64h ..] / 8 (fp32 [N x K]; K = hidden,
//                       N = heads; src W_k, src2 the pool query)
enum PackKind { kPackTranspose = 0, kPackTransposePair = 1, kPackColumnPair = 2, kPackCopy = 3, kPackPoolKeys = 4 };
struct PackJob {
    const void *src, *src2;
    const float *gain;
    void *dst;
    int K, N, kind, first_wg;
};
int pack_workgroups(PackJob *jobs, int n);
hipError_t launch_pack(const PackJob *jobs, int n, int workgroups, hipStream_t stream);

}  // namespace ube
