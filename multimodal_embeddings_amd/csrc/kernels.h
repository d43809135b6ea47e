// kernels.h -- launch interface of the gfx950 kernels of the encoder (internal to libube).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ube {

// Rows of every activation buffer past the last token; reads of a partial
// tile stay inside the allocation and see finite values.
constexpr int kRowPad = 256;
// Tokens per work tile of the gather, patchify and attention kernels.
constexpr int kTileTokens = 256;
// Partial sums of squares kept per token row (one per 64 features; D <= 1024).
constexpr int kSsParts = 16;

enum Epilogue : int {
    kEpiStore = 0,   // C = bf16(acc)                                   [M x N], ld
    kEpiQkv = 1,     // rotary on q, k -> qk [M x 2D]; v -> vt [D x ldvt] (feature-major)
    kEpiResid = 2,   // x[M x N] += acc (fp32)
    kEpiSwiglu = 3,  // interleaved gate/up blocks of 32 -> a = bf16(SiLU(g) * u)   [M x N/2]
    kEpiPatch = 4,   // x = acc * scale (fp32)
};

struct GemmArgs {
    const uint16_t *w;  // [N x K] bf16, K contiguous (packed weights)
    const uint16_t *x;  // [M_alloc x K] bf16 activations, M_alloc >= round_up(M, 256)
    int M, N, K;
    uint16_t *out_bf16;
    int ld_out;
    float *out_f32;
    int ld_f32;
    const float *res_in;  // residual: x read from here (ld_f32) and x + acc written to out_f32; NULL: in place
    uint16_t *gu_out;     // SwiGLU: when set, also the bf16 pre-activations [M x N] (interleaved as the product)
    int ld_gu;
    uint16_t *vt;
    int ld_vt;
    const int16_t *pos;   // [M_alloc x 4] rotary coordinates per token
    const float2 *rope;   // [positions x 32] (cos, sin)
    int D;                // width of q, k, v (QKV epilogue)
    int sec0, sec1;       // rotary pair sections: axis 0 for j < sec0, 1 for j < sec0+sec1, else 2
    float scale;          // patch epilogue scale
    const float *x_scale; // E4M3: per-token activation scale [M_alloc]
    float w_scale;        // E4M3: weight tensor scale (gate tensor for SwiGLU)
    float w_scale2;       // E4M3: up tensor scale (SwiGLU)
    float *ss_out;        // residual / patch: partial sums of squares of the new x [M_alloc x kSsParts], one
                          // per 256 features (N % 256 == 0 kernel) or per 64 (otherwise), and x's bf16 copy
                          // into out_bf16 (ld_out), when not NULL
    const float *ss_in;   // QKV / gate-up: scale rows by 1/sqrt(sum(ss_in[m][0..ss_parts)) / K + eps)
    int ss_parts;
    float eps;
};

hipError_t launch_gemm(int epilogue, const GemmArgs &args, hipStream_t stream);
// E4M3 operands (w, x are bytes; K counts elements, K % 128 == 0, N % 256 == 0);
// the accumulator is multiplied by x_scale[token] * w_scale before the epilogue.
hipError_t launch_gemm_e4m3(int epilogue, const GemmArgs &args, hipStream_t stream);

// Byte gather: x (fp32), its bf16 copy xb, the row's sum of squares (part 0 of
// kSsParts; the rest 0) and text positions. Tiles are (item, first token).
hipError_t launch_gather_text(const uint8_t *data, const int64_t *src, const int *cu, const int2 *tiles,
                              int ntiles, const uint16_t *embed, float *x, uint16_t *xb, float *ss, int16_t *pos,
                              int D, hipStream_t stream);

// Patch rows (bf16 [T x 768], values 0..255) and rotary coordinates.
struct MediaItem {
    int64_t pixel_offset;  // byte offset of the item in the tape data
    int frames, grid_h, grid_w, width;
};
hipError_t launch_patchify(const uint8_t *pixels, const MediaItem *items, const int *cu, const int2 *tiles,
                           int ntiles, uint16_t *patches, int16_t *pos, int axes, hipStream_t stream);

// E4M3 activations: codes + per-row scale amax/448 (value = code * scale).
hipError_t launch_rmsnorm_e4m3(const float *x, const float *gain, uint8_t *h8, float *hs, int T, int D, float eps,
                               hipStream_t stream);
hipError_t launch_quantize_rows(const uint16_t *in, uint8_t *out, float *scale, int T, int W, hipStream_t stream);

hipError_t launch_rmsnorm(const float *x, const float *gain, uint16_t *h, int T, int D, float eps,
                          hipStream_t stream);

// lse (optional, head-major [heads x ldl]): log2 of each query's softmax denominator in units of
// log2(e) q.k / 8, for the backward pass
hipError_t launch_attention(const uint16_t *q, const uint16_t *k, int ldqk, const uint16_t *vt, int ldvt,
                            uint16_t *o, int ldo, const int *cu, const int2 *tiles, int ntiles, int heads,
                            hipStream_t stream, float *lse = nullptr, int ldl = 0);

// Final RMSNorm -> xf (bf16) and pool scores s[t][h] = xf_t . u_h (fp32).
hipError_t launch_final_norm_scores(const float *x, const float *gain, const float *u, uint16_t *xf, float *s,
                                    float *states, int T, int D, int H, float eps, hipStream_t stream);
// rows of `in` [T x W] divided by their norms, into out as f32 or bf16
hipError_t launch_unit_rows(const float *in, void *out, int out_bf16, int T, int W, hipStream_t stream);
// hard MaxSim of every (query item, document item) pair; columns 128 or 256
hipError_t launch_maxsim(const uint16_t *q, const size_t *qoff, size_t qrows, size_t qld, int nq, const uint16_t *d,
                         const size_t *doff, size_t drows, size_t dld, int nd, int columns, size_t prefix, size_t span,
                         float *scores, size_t ld, hipStream_t stream);

// Per item: softmax of the scores over the item's tokens per head,
// z_h = sum_t p_t,h xf_t, pooled_h = z_h W_v[:, head h]; empty items -> 0.
// tiles: the 256-token tiles (item, first token); itile[count + 1]: first tile of each item.
// zp, zs: scratch of pool_partial_bytes / pool_stats_bytes.
size_t pool_partial_bytes(int ntiles, int D, int H);
size_t pool_stats_bytes(int ntiles, int H);
hipError_t launch_pool(const uint16_t *xf, const float *s, const int *cu, const int2 *tiles, int ntiles,
                       const int *itile, int count, const uint16_t *wv, void *out, int out_bf16, size_t out_stride,
                       int D, int H, float *zp, float2 *zs, hipStream_t stream);

}  // namespace ube
