// train.h -- launch interface of the gfx950 kernels of the encoder's backward pass and the Adafactor
// update (internal to libube).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ube {

// Attention backward for one head width of 64: rows of q, k (after the rotary), v, dO; the softmax log2
// denominators (lse, head-major, base-2 units of log2(e) q.k / 8) and delta = rowsum(dO * O) per query
// and head; tiles as the forward's (item, first token) list of 256-token tiles.
struct AttnBwdArgs {
    const uint16_t *q, *k;
    int ldqk;
    const uint16_t *v;
    int ldv;
    const uint16_t *dout;
    int lddo;
    const float *lse, *delta;
    int ldl;
    uint16_t *dq, *dk, *dv;  // rows [T x D]; dq, dk in the rotated space
    int ldd;
    const int *cu;
    const int2 *tiles;
    int ntiles;
    int heads;
};
hipError_t launch_attention_bwd(const AttnBwdArgs &a, hipStream_t stream);
// delta[h][t] = sum_e dO[t][64h + e] O[t][64h + e]
hipError_t launch_attention_delta(const uint16_t *dout, const uint16_t *o, int ld, float *delta, int ldl, int T,
                                  int heads, hipStream_t stream);
// v rows [T x D] from the feature-major vt [D x ldvt]
hipError_t launch_vt_rows(const uint16_t *vt, int ldvt, uint16_t *v, int T, int D, hipStream_t stream);
// Rotary backward (1-axis text positions pos[t * 4]): dqkv [T x 3D] = (R^T dq | R^T dk | dv)
hipError_t launch_rope_bwd(const uint16_t *dq, const uint16_t *dk, const uint16_t *dv, int ld, const int16_t *pos,
                           const float2 *rope, uint16_t *dqkv, int T, int D, hipStream_t stream);
// SwiGLU backward: gu [T x 2F] interleaved in blocks of 32 (gate | up), da [T x F] -> dgu (same interleave)
// and a = SiLU(g) u [T x F]
hipError_t launch_swiglu_bwd(const uint16_t *gu, const uint16_t *da, uint16_t *dgu, uint16_t *a, int T, int F,
                             hipStream_t stream);
// RMSNorm backward with residual: dx = dres + d/dx <rmsnorm(x) * g, dh>; dxb = bf16(dx) (optional);
// gain partials gpart[block][D] = sum over the block's rows of dh * x / rms (rows_per_block rows each)
hipError_t launch_rmsnorm_bwd(const float *x, const float *gain, const float *dh, const float *dres, float *dx,
                              uint16_t *dxb, float *gpart, int rows_per_block, int T, int D, float eps,
                              hipStream_t stream);
int rmsnorm_bwd_blocks(int T, int rows_per_block);
// out[m][n] = sum over t of X[t][m] Y[t][n] (bf16 operands, fp32 partials per split of t, then reduced);
// M % 128 == 0, N % 64 == 0. With `deinterleave`, n runs over [gate 32 | up 32] blocks and out receives
// the gate columns, out2 the up columns ([M x N/2] each).
hipError_t launch_xty(const uint16_t *x, int ldx, const uint16_t *y, int ldy, int T, int M, int N, float *partial,
                      int splits, int chunk, float *out, float *out2, bool deinterleave, hipStream_t stream);
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
// dz [count x H x D] and pd [T x H x 2] are work buffers
hipError_t launch_pool_bwd(const PoolBwdArgs &a, float *dz, float *pd, hipStream_t stream);

// Adafactor on one tensor: rows x cols (cols == 0: a vector of `rows`); g fp32; master bf16 (w16) or fp32
// (w32); state r [rows], c [cols] (matrices) or v [rows] (vectors), m [rows x cols]; work: kAdafactorWork +
// kAdafactorColParts floats. lr, beta2 and the bias correction 1 - beta1^t come from the host.
struct AdafactorArgs {
    const float *g;
    uint16_t *w16;
    float *w32;
    float *r, *c, *v, *m;
    float *work;
    int rows, cols;
    float lr, beta1, beta2, eps1, clip, bias_correction;
};
hipError_t launch_adafactor(const AdafactorArgs &a, hipStream_t stream);

// Packing for the forward: out[n][k] = bf16(W[k][n] * (gain ? gain[k] : 1)) for W [K x N] bf16; with
// `interleave`, W is the pair (W, W2) [K x N] each and out rows run over [W 32 | W2 32] blocks.
hipError_t launch_pack_transpose(const uint16_t *w, const uint16_t *w2, const float *gain, uint16_t *out, int K,
                                 int N, bool interleave, hipStream_t stream);
// out [K x 2N]: the columns of W and W2 [K x N] interleaved in blocks of 32 ([W 32 | W2 32] per 64)
hipError_t launch_interleave_cols(const uint16_t *w, const uint16_t *w2, uint16_t *out, int K, int N,
                                  hipStream_t stream);
// the pool's folded keys u_h = W_k[:, head h] q_h / 8 ([H x D] fp32)
hipError_t launch_pool_u(const uint16_t *wk, const uint16_t *query, float *u, int D, int H, hipStream_t stream);
constexpr int kAdafactorWork = 2 + 128;           // floats of AdafactorArgs::work before the column partials
constexpr size_t kAdafactorColParts = 1 << 18;   // column partials (ceil(rows / 32) x cols floats) after them

}  // namespace ube
