/*
 * ube.h -- C ABI of the MI355X (gfx950) forward pass of the uniform byte encoder.
 *
 * What is computed (UForm documentation pages):
 *   - "UForm" page, "Architecture & Goals": bytes in, N blocks at one fixed width
 *     (RMSNorm, QKV attention with multi-axis M-RoPE, SwiGLU MLP, residuals),
 *     an attention-pooled embedding out.
 *   - "UForm" page, "One Omni Model": byte-gather frontend for text, 16x16 patch
 *     projection with 2-D (row, col) rotary positions for images, and per-frame
 *     patches with 3-D (frame, row, col) positions for video.
 *   - "UForm" page, "Precision by Design": bf16 storage, fp32 accumulation and
 *     normalisation, fp32 residual stream; E4M3 inference fixed at load by one
 *     `quantization` argument, blocks in FP8, frontend and pool in bf16.
 *   - "UForm" page, FAQ "Why attention pooling instead of mean pooling?": the pool
 *     query is one learned vector of encoder width; per-token outputs are K and V.
 *
 * The call shapes follow the pages' C ABI:
 *   - "Arenas" page: one argument struct per verb with an `outcome` pointer;
 *     outputs land in a caller-reused arena that rewinds on every call and grows
 *     only when outgrown; rows views carry data, count, columns, stride, scalar;
 *     ragged inputs are Arrow tapes with count+1 offsets in host memory.
 *   - "Rust" and "Python" pages, "Encoding": `text_encode` takes a tape, a byte per
 *     token; `image_encode_pixels` takes interleaved 8-bit RGB with per-item
 *     heights and widths; outputs are f32 by default or bf16; stats count the
 *     items that were cut short and the tokens that were encoded.
 *   - "Python" page, "Errors": the status codes.
 *
 * Threading: calls on different arenas may run concurrently; one arena takes a
 * single call at once (a second, overlapping call reports `contended`). All device work
 * of a call is enqueued on the caller's HIP stream (`stream`, a hipStream_t; NULL
 * is the null stream).
 */
#ifndef UBE_H
#define UBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Outcome of a call ("Python" page, "Errors"; subset used by the encoder). */
typedef enum ube_status_t {
    ube_status_success_k = 0,
    ube_status_invalid_argument_k = 1, /* NULL arena or argument, decreasing offsets, inputs inside the arena */
    ube_status_shape_mismatch_k = 2,   /* image side not a multiple of the patch, patches over the context */
    ube_status_out_of_memory_k = 3,    /* the GPU could not grow the arena; no host fallback */
    ube_status_device_k = 4,           /* arena and model on different devices, or a HIP runtime failure */
    ube_status_contended_k = 5,        /* the arena is serving another call */
    ube_status_unsupported_k = 6,      /* a geometry or mode the library does not run */
    ube_status_internal_k = 7,
} ube_status_t;

/* `message` is a static string, never freed; NULL on success. */
typedef struct ube_outcome_t {
    ube_status_t status;
    char const *message;
} ube_outcome_t;

typedef enum ube_scalar_t {
    ube_scalar_unknown_k = 0,
    ube_scalar_u8_k = 1,
    ube_scalar_bf16_k = 2,
    ube_scalar_f32_k = 3,
    ube_scalar_e4m3_k = 4,
} ube_scalar_t;

/* Ragged input, Arrow layout ("Arenas" page, "Rows and Tapes"): item i spans
 * data[offsets[i] .. offsets[i+1]). `offsets` (count+1 entries) is host memory;
 * `data` may be device memory of the model's GPU (used in place) or host memory
 * (copied to the device by the call). offsets[0] may be non-zero. */
typedef struct ube_tape_view_t {
    void const *data;
    size_t const *offsets;
    size_t count;
} ube_tape_view_t;

/* Output rows, one per item ("Arenas" page, "Rows and Tapes"): row i starts at
 * (char*)data + i*stride and holds `columns` values of `scalar`. Device memory
 * inside the arena, valid until the next call naming that arena. */
typedef struct ube_rows_view_t {
    void *data;
    size_t count, columns, stride;
    ube_scalar_t scalar;
} ube_rows_view_t;

/* Ragged output rows ("Arenas" page, "Rows and Tapes": rows packed back to back,
 * count + 1 offsets): item i owns rows offsets[i] .. offsets[i+1]; row r
 * starts at (char*)data + r*stride and holds `columns` values of `scalar`;
 * `rows` = offsets[count]. Written by an encode, data and offsets are device
 * memory inside the arena, valid until the next call naming that arena. */
typedef struct ube_rows_tape_view_t {
    void *data;
    size_t const *offsets;
    size_t count, rows, columns, stride;
    ube_scalar_t scalar;
} ube_rows_tape_view_t;

/* Surfaces an encode writes ("Rust" and "Python" pages, "Encoding": Outputs);
 * OR-ed together, 0 meaning embeddings alone. States are the final-norm rows,
 * one per token; token vectors are the unit-normalised outputs of the token head, on the same
 * offsets. A surface left out costs nothing past the final norm. */
typedef enum ube_outputs_t {
    ube_outputs_embeddings_k = 1,
    ube_outputs_states_k = 2,
    ube_outputs_token_vectors_k = 4,
} ube_outputs_t;

/* "Python" page, "Encoding": items cut at the context, and tokens encoded. */
typedef struct ube_encode_stats_t {
    size_t truncated, tokens;
} ube_encode_stats_t;

/* Model shape. Zero fields take the default in brackets.
 * depth N [required], hidden D [required, multiple of 128], heads H [D/64; D/H
 * must be 64], ffn F [3D; multiple of 64], vocab [258], context [1024; at most
 * 32767], rope_axes [1; 1 text, 2 image, 3 video], patch_side [16], channels
 * [3], rope_base [10000], rms_epsilon [1e-6], quantization [bf16; or e4m3],
 * token_width [0 = no token head; a multiple of 128 up to 1024 here, where the
 * pages allow multiples of 8; "Training" page, uform_late_interaction_t]. */
typedef struct ube_geometry_t {
    size_t depth, hidden, heads, ffn, vocab, context, rope_axes, patch_side, channels;
    float rope_base, rms_epsilon;
    ube_scalar_t quantization;
    size_t token_width;
} ube_geometry_t;

/* Weights in host memory, canonical layout y = x W with W row-major [in x out].
 * Matrices are bf16 bit patterns (uint16); gains are float32. Per-block arrays
 * hold `depth` pointers. The model copies and packs everything at init; the
 * caller may free these afterwards.
 *   embed      [vocab x D]          text models (NULL for media)
 *   patch_proj [p*p*channels x D]   media models (NULL for text)
 *   w_qkv      [D x 3D] = [W_q | W_k | W_v];  w_o [D x D]
 *   w_gate, w_up [D x F];  w_down [F x D]
 *   attn_norm, mlp_norm, final_norm: [D]
 *   pool_query [D];  pool_wk, pool_wv [D x D]
 *   token_head [D x token_width] (NULL when token_width is 0): the per-token
 *   projection whose rows, divided by their norms, are the token vectors */
typedef struct ube_weights_t {
    uint16_t const *embed;
    uint16_t const *patch_proj;
    uint16_t const *const *w_qkv;
    uint16_t const *const *w_o;
    uint16_t const *const *w_gate;
    uint16_t const *const *w_up;
    uint16_t const *const *w_down;
    float const *const *attn_norm;
    float const *const *mlp_norm;
    float const *final_norm;
    uint16_t const *pool_query;
    uint16_t const *pool_wk;
    uint16_t const *pool_wv;
    uint16_t const *token_head;
} ube_weights_t;

typedef struct ube_model_handle_t *ube_model_t;
typedef struct ube_arena_handle_t *ube_arena_t;

/* Loads a model onto GPU `device`: validates the geometry, packs the weights
 * for the gfx950 kernels (and quantises the block matrices to E4M3 with one
 * amax/448 scale per tensor when geometry.quantization is e4m3), and builds
 * the rotary cos/sin table (double on the host, stored fp32). On failure
 * *model is NULL. Statuses: invalid_argument (NULL or missing weights),
 * unsupported (geometry outside the bounds above), out_of_memory, device. */
typedef struct ube_model_init_t {
    ube_model_t *model;
    ube_outcome_t *outcome;
    int device;
    ube_geometry_t geometry;
    ube_weights_t const *weights;
} ube_model_init_t;
void ube_model_init(ube_model_init_t *arguments);

typedef struct ube_model_description_t {
    size_t dimensions, context, depth, heads, ffn, rope_axes;
    ube_scalar_t quantization;
    size_t memory_usage; /* device bytes the model holds */
    int device;
    size_t token_width;  /* 0: the model has no token head */
} ube_model_description_t;

typedef struct ube_model_describe_t {
    ube_model_t model;
    ube_outcome_t *outcome;
    ube_model_description_t *description;
} ube_model_describe_t;
void ube_model_describe(ube_model_describe_t *arguments);

/* NULL-safe; cannot fail. Waits for nothing: the caller finishes its streams first. */
void ube_model_free(ube_model_t model);

/* An empty arena on GPU `device` ("Arenas" page, `uform_arena_init`): it holds
 * no memory before the first call that writes into it. Here the arena also holds
 * the call's activations, so an arena is the unit of concurrency.
 * capacity_limit: device bytes the arena may grow to (0: no limit). A call that
 * would need more fails with out_of_memory and NULL outputs, as when the GPU has
 * no memory left ("Python" page, "Errors"); the arena keeps what it held. */
typedef struct ube_arena_init_t {
    ube_arena_t *arena;
    ube_outcome_t *outcome;
    int device;
    size_t capacity_limit;
} ube_arena_init_t;
void ube_arena_init(ube_arena_init_t *arguments);

/* NULL-safe; synchronises the device, then frees the arena and its outputs. */
void ube_arena_free(ube_arena_t arena);

/* Device bytes the arena holds now (its high-water mark). */
size_t ube_arena_capacity(ube_arena_t arena);

/* Encodes a tape of byte strings, a byte per token ("Rust"/"Python" pages,
 * `text_encode`). Items longer than the model context keep their first
 * `context` bytes and count in stats->truncated. Writes one pooled row of D
 * values per item into the arena as `outputs_scalar` (f32, the default when
 * unknown, or bf16) and publishes it through *embeddings; an item with no
 * bytes pools to the zero row; count == 0 succeeds with an empty view.
 * completion == 0 blocks until the rows are final; 1 returns once the work is
 * queued on `stream` (a GPU fault then surfaces at the caller's next
 * synchronisation). On failure *embeddings is all zeros and NULL.
 * `trace_residual`, when not NULL, is device memory of (depth+1) * T * D
 * floats that receives the fp32 residual stream after the frontend and after
 * every block (T = stats->tokens): a diagnostics hook, off the timed path.
 * `outputs` (ube_outputs_t bits, 0 = embeddings) picks the surfaces: with
 * states, *states receives the final-norm rows [T x D]; with token vectors,
 * *token_vectors receives the unit rows [T x token_width] (unsupported when the
 * model has no token head); both on the offsets of the kept tokens, as
 * `outputs_scalar`. A surface not asked for is published empty; its pointer
 * may then be NULL. */
typedef struct ube_text_encode_t {
    ube_model_t model;
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_tape_view_t texts;
    ube_scalar_t outputs_scalar;
    ube_rows_view_t *embeddings;
    ube_encode_stats_t *stats;
    float *trace_residual;
    unsigned outputs;
    ube_rows_tape_view_t *states;
    ube_rows_tape_view_t *token_vectors;
} ube_text_encode_t;
void ube_text_encode(ube_text_encode_t *arguments);

/* Encodes images of interleaved 8-bit RGB ("Rust"/"Python" pages,
 * `image_encode_pixels`): item i is heights[i] x widths[i] x channels bytes of
 * the tape, cut into patch_side^2 patches in row-major grid order, each patch
 * vector ordered (row in patch, column in patch, channel) and scaled by 1/255,
 * projected by patch_proj; positions (grid row, grid col) on a 2-axis model.
 * heights/widths are host arrays of `count`. shape_mismatch when a side is not
 * a multiple of patch_side, the item's bytes differ from its size, or its patch
 * count exceeds the context. Otherwise as ube_text_encode. */
typedef struct ube_image_encode_pixels_t {
    ube_model_t model;
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_tape_view_t pixels;
    size_t const *heights;
    size_t const *widths;
    ube_scalar_t outputs_scalar;
    ube_rows_view_t *embeddings;
    ube_encode_stats_t *stats;
    float *trace_residual;
    unsigned outputs;
    ube_rows_tape_view_t *states;
    ube_rows_tape_view_t *token_vectors;
} ube_image_encode_pixels_t;
void ube_image_encode_pixels(ube_image_encode_pixels_t *arguments);

/* Extension (the pages offer video only from files): item i is frame_counts[i]
 * frames of heights[i] x widths[i] x channels bytes, each frame cut into
 * patches as for images; token (f, r, c) sits at f*gh*gw + r*gw + c with
 * positions (frame, row, col) on a 3-axis model. Otherwise as images. */
typedef struct ube_video_encode_frames_t {
    ube_model_t model;
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_tape_view_t frames;
    size_t const *frame_counts;
    size_t const *heights;
    size_t const *widths;
    ube_scalar_t outputs_scalar;
    ube_rows_view_t *embeddings;
    ube_encode_stats_t *stats;
    float *trace_residual;
    unsigned outputs;
    ube_rows_tape_view_t *states;
    ube_rows_tape_view_t *token_vectors;
} ube_video_encode_frames_t;
void ube_video_encode_frames(ube_video_encode_frames_t *arguments);

/* Hard MaxSim scores ("UForm" page, the reranker paragraph of its losses: each
 * query token keeps its best inner product over the candidate's tokens,
 * averaged over the query). scores[i * scores_stride + j] = mean over query i's
 * rows t in [prefix, prefix + span) (clipped to the item) of max over document
 * j's rows s of <q_t, d_s>; a query with no counted rows, or an empty document,
 * scores 0. query_span 0 means 64, the pages' max_query_span ("Training" page,
 * uform_late_interaction_t). Both tapes are bf16 rows of the same `columns`
 * (a multiple of 16, at most 1024) in device memory of `device`, offsets
 * included (as an encode's token vectors are); offsets past `rows` are clamped
 * to it. `scores` is device memory, scores_stride 0 meaning documents.count.
 * completion == 0 blocks until the scores are final. invalid_argument on NULL
 * or mismatched inputs; unsupported for other scalars or widths. */
typedef struct ube_maxsim_t {
    void *stream;
    ube_outcome_t *outcome;
    int device;
    int completion;
    ube_rows_tape_view_t queries;
    ube_rows_tape_view_t documents;
    size_t query_prefix, query_span;
    float *scores;
    size_t scores_stride;
} ube_maxsim_t;
void ube_maxsim(ube_maxsim_t *arguments);

/* Negative pairs of the contrastive loss ("Training" page, uform_negatives_t): ambient repels
 * every pair no edge names at `ambient_repulsion_weight` (and the named repel edges); named repels the
 * repel edges alone. */
typedef enum ube_negatives_t {
    ube_negatives_ambient_k = 0,
    ube_negatives_named_k = 1,
} ube_negatives_t;

/* How a row of scores turns into forces ("Training" page, uform_pair_loss_form_t). This library runs
 * the sigmoid form (SigLIP's, the pooled embeddings' own); balanced and ranked report unsupported. */
typedef enum ube_pair_loss_form_t {
    ube_pair_loss_form_derived_k = 0,
    ube_pair_loss_form_balanced_k = 1,
    ube_pair_loss_form_ranked_k = 2,
    ube_pair_loss_form_sigmoid_k = 3,
} ube_pair_loss_form_t;

/* One edge set over the anchors in compressed rows ("Training" page, uform_edges_view_t): anchor p
 * links to items ids[offsets[p] .. offsets[p+1]), strictly ascending within each run; `weights`, when
 * not NULL, pairs a weight with each id (else every edge weighs 1; ignore edges read none). Host
 * memory; offsets NULL names no edges, otherwise it has anchor_count + 1 entries. */
typedef struct ube_edges_view_t {
    size_t const *offsets;
    uint32_t const *ids;
    float const *weights;
} ube_edges_view_t;

/* The contrastive targets ("Training" page, uform_relations_view_t), resolved per pair in the pages'
 * order: ignore skips, attract pulls, repel pushes, every other pair follows `negatives`. */
typedef struct ube_relations_view_t {
    ube_edges_view_t attract, repel, ignore;
} ube_relations_view_t;

/* Matryoshka sigmoid contrastive loss over pooled embeddings, forward and backward ("UForm" page,
 * "Matryoshka-Like Multi-Scale Embedders": every nested prefix width scored under SigLIP's per-cell
 * sigmoid loss; "Training" page, uform_contrastive_t for the widths, inverse temperature, bias and
 * ambient weight). The step's `count` items are bf16 rows of `columns` (a multiple of 64, at most 4096)
 * in device memory of the arena's GPU; anchors are items [anchor_begin, anchor_begin + anchor_count) (one
 * device's share of a gathered band), every item is a candidate, and an item paired with itself is
 * skipped. For each width m: cosine s of the length-m prefixes (a zero prefix has cosine 0), logit
 * z = inverse_temperature * s + bias, cell loss -w log sigma(z) for an attract edge of weight w and
 * -w log(1 - sigma(z)) for a repelled pair; the width's loss sums the cells of an anchor's row and
 * averages over anchors, and the loss is the mean over widths.
 * `matryoshka_dimensions`: host array of strictly ascending widths, each a multiple of 8 up to `columns`,
 * at most 8 (NULL: `columns` alone); this library runs multiples of 64 and reports others unsupported.
 * Outputs (device memory): `scalars` receives 3 + widths floats: the loss, d loss / d inverse_temperature,
 * d loss / d bias, then each width's loss (the loss entries are NaN when `want_loss` is 0, which skips
 * their per-pair logarithms). `gradient`, when not NULL, receives d loss / d embedding as fp32 rows of
 * `columns` at `gradient_stride` bytes (16-byte aligned); columns past the widest width get 0.
 * The arena is the call's workspace (it grows to about 2 * widths * anchors * count bytes plus small
 * buffers and invalidates earlier views into it); the embeddings must not lie in it. completion == 0
 * blocks until the outputs are final. Statuses: invalid_argument (NULL or misaligned pointers, anchors
 * outside the items, bad widths or edges), unsupported (non-bf16 rows, other widths or loss forms),
 * contended, device, out_of_memory. */
typedef struct ube_contrastive_t {
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_rows_view_t embeddings;
    size_t anchor_begin, anchor_count;
    size_t const *matryoshka_dimensions;
    size_t matryoshka_dimensions_count;
    float inverse_temperature, bias;
    ube_negatives_t negatives;
    float ambient_repulsion_weight;
    ube_pair_loss_form_t pair_loss;
    ube_relations_view_t relations;
    int want_loss;
    float *scalars;
    float *gradient;
    size_t gradient_stride;
} ube_contrastive_t;
void ube_contrastive(ube_contrastive_t *arguments);

/* Training of a text model ("UForm" page, "Precision by Design" and "Adafactor Optimizer"; "Training"
 * page, uform_trainer_t and uform_trainer_step: forward, loss, backward, update). One device; the loss is
 * the caller's (for example ube_contrastive over the pooled rows), handed in as its gradient with respect
 * to the pooled embeddings.
 *
 * A trainer keeps bf16 master weights (fp32 for the norm gains) in the canonical layout of ube_weights_t,
 * their fp32 gradients and the Adafactor state, and refreshes the model's forward weights after every
 * step (so encodes on the model see the updated weights). Text models in bf16 with 1-axis rotary,
 * hidden a multiple of 128 up to 1024 and ffn a multiple of 128 (unsupported otherwise). Adafactor: beta1 [0.9], decay_rate [-0.8] (beta2_t = 1 -
 * t^decay_rate), epsilon1 [1e-30], clip_threshold [1]; zero fields take the defaults in brackets; the
 * update reads each fp32 gradient cast to bf16 (nearest even). With activation_recomputation the
 * training forward keeps only every block's fp32 input and the backward replays each block's attention
 * half from it (the pages' memory plan: 4 * hidden bytes per token and block); without it the forward
 * keeps what the backward reads (about 16 * hidden + 4 * ffn bytes per token and block, no replay). */
typedef struct ube_trainer_handle_t *ube_trainer_t;

typedef struct ube_trainer_init_t {
    ube_trainer_t *trainer;
    ube_outcome_t *outcome;
    ube_model_t model;               /* borrowed until the trainer is freed */
    ube_weights_t const *weights;    /* the model's weights in host memory (copied) */
    float beta1, decay_rate, epsilon1, clip_threshold;
    int activation_recomputation;    /* nonzero: keep only each block's fp32 input ("Precision by Design") */
} ube_trainer_init_t;
void ube_trainer_init(ube_trainer_init_t *arguments);

/* Training forward over a byte tape: the model's forward, with the activations its backward reads kept in
 * the trainer's device memory (per block: the fp32 input; without recomputation also the fp32 rows after
 * the attention half, the rotated q|k rows, v, the attention output and its softmax denominators, and
 * the gate/up pre-activations).
 * *embeddings receives the pooled fp32 rows [count x hidden] in the arena, valid until
 * the arena's next call. The kept activations serve the next ube_trainer_backward with after_forward set,
 * until a step changes the weights. */
typedef struct ube_trainer_forward_t {
    ube_trainer_t trainer;
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_tape_view_t texts;
    ube_rows_view_t *embeddings;
    ube_encode_stats_t *stats;
} ube_trainer_forward_t;
void ube_trainer_forward(ube_trainer_forward_t *arguments);

/* Backward pass: walks the blocks from last to first over the kept activations (replaying each block's
 * attention half first under recomputation), rebuilding each block's two RMSNorm outputs, v's rows and
 * the gate/up pre-activations. after_forward != 0:
 * differentiates the rows of the last ube_trainer_forward (arena, texts and stats unused; an error if a
 * step came in between); after_forward == 0: runs that forward over `texts` on `arena` first.
 * d_embeddings: device fp32 rows [count x hidden] (packed; stride 0 or hidden * 4 bytes), d loss / d
 * pooled embedding. Writes d loss / d every parameter into the trainer's fp32 gradient buffers
 * (overwritten, not accumulated). */
typedef struct ube_trainer_backward_t {
    ube_trainer_t trainer;
    ube_arena_t arena;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    ube_tape_view_t texts;
    float const *d_embeddings;
    size_t d_embeddings_stride;
    ube_encode_stats_t *stats;
    int after_forward;
} ube_trainer_backward_t;
void ube_trainer_backward(ube_trainer_backward_t *arguments);

/* One Adafactor update of every tensor with the gradients of the last backward, at `learning_rate`
 * (the caller's schedule); then the model's forward weights are rebuilt from the masters. */
typedef struct ube_trainer_step_t {
    ube_trainer_t trainer;
    void *stream;
    ube_outcome_t *outcome;
    int completion;
    float learning_rate;
} ube_trainer_step_t;
void ube_trainer_step(ube_trainer_step_t *arguments);

/* Device views of the trainer's tensors, in a fixed order (embed; per block attn_norm, w_qkv, w_o,
 * mlp_norm, w_gate, w_up, w_down; final_norm, pool_query, pool_wk, pool_wv): canonical layout, `cols` 0
 * for vectors; master bf16 or f32; gradient fp32. Returns the tensor count; fills at most `capacity`. */
typedef struct ube_trainer_tensor_t {
    char const *name;
    size_t layer, rows, cols;
    void *master;
    ube_scalar_t master_scalar;
    float *gradient;
} ube_trainer_tensor_t;
size_t ube_trainer_tensors(ube_trainer_t trainer, ube_trainer_tensor_t *tensors, size_t capacity);

/* NULL-safe; synchronises the device, then frees the trainer's memory. */
void ube_trainer_free(ube_trainer_t trainer);

/* Host-only tape plan, the bookkeeping every text encode does first (no
 * device work; usable without a GPU). lengths[count] receives the kept length
 * of each item, cu[count+1] their prefix sums, *stats the truncated items and
 * tokens. Returns invalid_argument if an offset decreases or a pointer is NULL
 * with count > 0. */
ube_status_t ube_tape_plan(size_t const *offsets, size_t count, size_t context, uint32_t *lengths, uint32_t *cu,
                           ube_encode_stats_t *stats);

/* Spelling of a status, a static string. */
char const *ube_status_name(ube_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* UBE_H */
