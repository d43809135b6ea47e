/*
 * ube_steps.h -- per-step entry points and kernel timing of libube.
 *
 * Each step entry point launches one kernel of the encode path on device
 * buffers the caller owns, so every step of the forward pass can be checked
 * on its own against a CPU reference. They use the library's internal layouts,
 * stated with each call. All pointers are device memory of the current device
 * unless noted; `stream` is a hipStream_t (NULL: null stream). Each returns
 * invalid_argument for NULL pointers or unsupported sizes, device for a HIP
 * runtime failure, success otherwise; the work is asynchronous on `stream`
 * unless noted.
 */
#ifndef UBE_STEPS_H
#define UBE_STEPS_H

#include <stddef.h>
#include <stdint.h>

#include "ube.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Projection ("UForm" page, "Architecture & Goals": the block's matrix
 * products, bf16 in, fp32 accumulate, "Precision by Design"):
 * y[M x N] = bf16(x[M x K] w^T), w given transposed as [N x K] (the packed
 * weight layout), all row-major bf16. x must have round_up(M, 256) readable
 * rows (rows past M are read, their products discarded). N % 128 == 0,
 * K % 64 == 0. */
ube_status_t ube_step_gemm(void const *w, void const *x, void *y, size_t M, size_t N, size_t K, void *stream);

/* RMSNorm ("UForm" page, "Architecture & Goals"; fp32 normalisation,
 * "Precision by Design"): h[t] = bf16(x[t] * gain / sqrt(mean(x[t]^2) + eps)),
 * x fp32 [T x D], gain fp32 [D], h bf16 [T x D]. */
ube_status_t ube_step_rmsnorm(float const *x, float const *gain, void *h, size_t T, size_t D, float eps,
                              void *stream);

/* Bidirectional variable-length attention ("UForm" page, FAQ "Why no cuDNN,
 * FlashAttention, xformers, or FA3?": ragged attention, each segment on its
 * own), head width 64: for every item i (tokens cu[i] .. cu[i+1]) and head h,
 * o_t,h = sum_u softmax_u(q_t,h . k_u,h / 8) v_u,h over u in item i.
 * q, k: bf16, row t at q + t*ldqk (elements), head h at columns [64h, 64h+64);
 * vt: bf16 feature-major, element (64h + e, t) at vt[(64h + e)*ldvt + t];
 * o: bf16, row t at o + t*ldo. cu_host: host, count+1 non-decreasing entries.
 * q and k need cu[count] + 256 readable rows, vt ldvt >= cu[count] + 256, with
 * columns cu[count] .. cu[count]+64 finite. Synchronous (allocates and frees
 * its tile list). */
ube_status_t ube_step_attention(void const *q, void const *k, size_t ldqk, void const *vt, size_t ldvt, void *o,
                                size_t ldo, uint32_t const *cu_host, size_t count, size_t heads, void *stream);

/* The attention step above for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not call hipMalloc): same
 * arguments, same kernel, same results bit for bit. The item bounds and the
 * 256-token tile list go to a fixed 1 MiB buffer the library holds on every GPU it
 * runs on (a static device array, kept until the process ends) instead of memory
 * allocated per call; it calls no hipMalloc, hipFree or hipHostMalloc. Limits:
 * count + 2 + 2 * tiles <= 262144 (tiles = sum over items of ceil(length / 256)),
 * else invalid_argument with nothing launched. Every call on one GPU shares that
 * buffer: calls that overlap on one GPU race (this call waits for `stream` before
 * it returns, so calls made one after another are safe). Synchronous. */
ube_status_t ube_step_attention_static(void const *q, void const *k, size_t ldqk, void const *vt, size_t ldvt,
                                       void *o, size_t ldo, uint32_t const *cu_host, size_t count, size_t heads,
                                       void *stream);

/* E4M3 activation rows ("UForm" page, "Precision by Design": an e4m3 model runs
 * its blocks in Float8): in bf16 [T x W] -> codes [T x W] (OCP E4M3FN bytes) and
 * scales[T] = amax_row / 448, code = nearest-even E4M3 of value * (448 / amax_row)
 * computed in fp32; an all-zero row gets scale 0 and zero codes. W % 8 == 0. */
ube_status_t ube_step_quantize_e4m3(void const *in, void *codes, float *scales, size_t T, size_t W, void *stream);

/* E4M3 projection: y[M x N] = bf16(sum_k (x[m,k] x_scale[m]) (w[n,k] w_scale)),
 * w codes [N x K], x codes with round_up(M, 256) readable rows and x_scale
 * entries. N % 256 == 0, K % 128 == 0. */
ube_status_t ube_step_gemm_e4m3(void const *w, float w_scale, void const *x, float const *x_scale, void *y, size_t M,
                                size_t N, size_t K, void *stream);

/* QKV projection with multi-axis rotary ("UForm" page, "Architecture & Goals": QKV
 * attention with M-RoPE; "One Omni Model": 1-D text, 2-D (row, col) image and 3-D
 * (frame, row, col) video coordinates), the kernel and epilogue an encode runs:
 * [q | k | v] = x w^T with w given transposed as [3D x K] (rows 0..D-1 give q,
 * D..2D-1 give k, 2D..3D-1 give v); accumulation fp32. Within every head of 64
 * features, pair j (features 2j, 2j+1) of q and k turns by the angle
 * pos[t][axis(j)] * base^(-2j/64); the 32 pairs form `rope_axes` contiguous sections
 * as even as possible, leading sections taking the remainder ([32]; [16, 16];
 * [11, 11, 10]). Outputs: qk bf16 [M x 2D] (row t = rotated q_t | rotated k_t),
 * vt bf16 feature-major [D x ldvt] (element (f, t) = v_t[f]; columns M ..
 * round_up(M, 256) - 1 are written as 0).
 * x: bf16 [M x K] with round_up(M, 256) readable rows (rows past M are read, their
 * products discarded). pos_host: host int16 [M x 4], entries 0..2 the token's
 * coordinates on axes 0..2, each in [0, positions); entry 3 unused.
 * Requirements: D % 128 == 0, K % 64 == 0, 1 <= rope_axes <= 3, positions <= 32767,
 * ldvt >= round_up(M, 256); invalid_argument otherwise or for a coordinate outside
 * [0, positions). Synchronous: builds the cos/sin table (double, stored fp32) and
 * uploads the coordinates into device memory it allocates and frees. */
ube_status_t ube_step_qkv_rotary(void const *w, void const *x, size_t M, size_t D, size_t K, int16_t const *pos_host,
                                 size_t rope_axes, float rope_base, size_t positions, void *qk, void *vt, size_t ldvt,
                                 void *stream);

/* Kernels of an encode, contrastive or trainer call, for timing. */
typedef enum ube_kernel_t {
    ube_kernel_gather_k = 0,
    ube_kernel_patchify_k = 1,
    ube_kernel_rmsnorm_k = 2,
    ube_kernel_gemm_patch_k = 3,
    ube_kernel_gemm_qkv_k = 4,
    ube_kernel_attention_k = 5,
    ube_kernel_gemm_out_k = 6,
    ube_kernel_gemm_gate_up_k = 7,
    ube_kernel_gemm_down_k = 8,
    ube_kernel_final_norm_k = 9,
    ube_kernel_pool_k = 10,
    ube_kernel_quantize_k = 11,
    ube_kernel_contrastive_cells_k = 12, /* contrastive loss: dense cells */
    ube_kernel_contrastive_rows_k = 13,  /* contrastive loss: rows contraction */
    ube_kernel_contrastive_cols_k = 14,  /* contrastive loss: columns contraction */
    ube_kernel_attention_bwd_k = 15,     /* trainer: attention backward (dQ, then dK and dV) */
    ube_kernel_weight_grad_k = 16,       /* trainer: weight gradients X^T Y */
    ube_kernel_count_k = 17,
} ube_kernel_t;

/* Starts timing every launch of `kernel` made by encode calls in this
 * process: a HIP event pair is recorded around each launch on the call's
 * stream, for at most `max_launches` launches (further ones go untimed).
 * Process-wide; one kernel at a time. Allocates the events now, none later. */
ube_status_t ube_kernel_timer_start(ube_kernel_t kernel, size_t max_launches);

/* Waits for the recorded events, returns the summed duration in milliseconds
 * and the number of timed launches, and stops timing (events are freed). */
ube_status_t ube_kernel_timer_stop(double *total_ms, size_t *launches);

/* Spelling of a kernel id, a static string. */
char const *ube_kernel_name(ube_kernel_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* UBE_STEPS_H */
