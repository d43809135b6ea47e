// engine.cpp -- host side of libube: model packing, arenas, tape plans, the
// launch sequence of an encode call, and the C ABI (include/ube.h,
// include/ube_steps.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "contrastive.h"
#include "kernels.h"
#include "train.h"
#include "ube.h"
#include "ube_steps.h"

using namespace ube;

namespace {

// ------------------------------------------------------------------ outcome

void set_outcome(ube_outcome_t *outcome, ube_status_t status, char const *message) {
    if (outcome) {
        outcome->status = status;
        outcome->message = status == ube_status_success_k ? nullptr : message;
    }
}

struct Failure {
    ube_status_t status;
    char const *message;
};

#define UBE_HIP(call)                                                                         \
    do {                                                                                      \
        hipError_t _e = (call);                                                               \
        if (_e != hipSuccess) {                                                               \
            if (_e == hipErrorOutOfMemory) throw Failure{ube_status_out_of_memory_k, "GPU out of memory"}; \
            throw Failure{ube_status_device_k, "HIP runtime error in " #call};                \
        }                                                                                     \
    } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------- kernel timer

struct KernelTimer {
    std::mutex mu;
    int kernel = -1;
    std::vector<hipEvent_t> events;  // pairs
    size_t used = 0;
};
KernelTimer g_timer;

// Launch `fn` (returns hipError_t) on `stream`, bracketed by events when `kernel` is being timed.
template <typename Fn>
void timed(ube_kernel_t kernel, hipStream_t stream, Fn fn) {
    hipEvent_t begin = nullptr, end = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_timer.mu);
        if (g_timer.kernel == (int)kernel && g_timer.used + 2 <= g_timer.events.size()) {
            begin = g_timer.events[g_timer.used];
            end = g_timer.events[g_timer.used + 1];
            g_timer.used += 2;
        }
    }
    if (begin) UBE_HIP(hipEventRecord(begin, stream));
    UBE_HIP(fn());
    if (end) UBE_HIP(hipEventRecord(end, stream));
}

}  // namespace

// ===================================================================== model

struct ube_model_handle_t {
    int device = 0;
    ube_geometry_t g{};
    bool text = true;
    char *mem = nullptr;
    size_t bytes = 0;
    uint16_t *embed = nullptr, *patch_t = nullptr, *wv = nullptr;
    struct Layer {
        uint16_t *wqkv, *wo, *wgu, *wd;  // packed [out x in]; E4M3 codes (bytes) when e4m3
        float *g1, *g2;
        float s_qkv = 1.f, s_o = 1.f, s_gate = 1.f, s_up = 1.f, s_down = 1.f;  // E4M3 tensor scales
    };
    bool e4m3 = false;
    std::vector<Layer> layers;
    float *gf = nullptr, *u = nullptr;
    float2 *rope = nullptr;
    uint16_t *tok = nullptr;  // token head, packed [token_width x D]
    int sec0 = 32, sec1 = 0;
};

namespace {

bool row_width_supported(size_t D) {
    if (D % 128 != 0 || D == 0) return false;
    if (D % 512 == 0) return D / 512 <= 4;
    if (D % 256 == 0) return (D / 256) % 2 == 1 && D / 256 <= 7;
    return (D / 128) % 2 == 1 && D / 128 <= 7;
}

ube_geometry_t complete_geometry(ube_geometry_t g) {
    if (!g.heads && g.hidden) g.heads = g.hidden / 64;
    if (!g.ffn) g.ffn = 3 * g.hidden;
    if (!g.vocab) g.vocab = 258;
    if (!g.context) g.context = 1024;
    if (!g.rope_axes) g.rope_axes = 1;
    if (!g.patch_side) g.patch_side = 16;
    if (!g.channels) g.channels = 3;
    if (g.rope_base == 0.f) g.rope_base = 10000.f;
    if (g.rms_epsilon == 0.f) g.rms_epsilon = 1e-6f;
    if (g.quantization == ube_scalar_unknown_k) g.quantization = ube_scalar_bf16_k;
    return g;
}

char const *check_geometry(ube_geometry_t const &g) {
    if (!g.depth) return "depth must be positive";
    if (!row_width_supported(g.hidden) || g.hidden > 1024) return "hidden must be a supported multiple of 128, <= 1024";
    if (g.heads * 64 != g.hidden) return "head width must be 64";
    if (g.heads > 16) return "at most 16 heads";
    if (g.ffn % 64 != 0) return "ffn must be a multiple of 64";
    if (g.context > 32767) return "context must be at most 32767";
    if (g.rope_axes < 1 || g.rope_axes > 3) return "rope_axes must be 1, 2 or 3";
    if (g.quantization != ube_scalar_bf16_k && g.quantization != ube_scalar_e4m3_k)
        return "quantization must be bf16 or e4m3";
    if (g.quantization == ube_scalar_e4m3_k && (g.hidden % 256 != 0 || g.ffn % 128 != 0))
        return "e4m3 blocks need hidden % 256 == 0 and ffn % 128 == 0";
    if (g.vocab > 65535) return "vocab too large";
    if (g.token_width && (!row_width_supported(g.token_width) || g.token_width > 1024))
        return "token_width must be a supported multiple of 128, <= 1024";
    return nullptr;
}

// dst[c * rows + r] = src[r * cols + c]  (transpose a row-major [rows x cols] matrix)
void transpose_into(uint16_t *dst, uint16_t const *src, size_t rows, size_t cols) {
    for (size_t r = 0; r < rows; ++r)
        for (size_t c = 0; c < cols; ++c) dst[c * rows + r] = src[r * cols + c];
}

float bf16_value(uint16_t b) {
    uint32_t w = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &w, 4);
    return f;
}

// float -> bf16 bits, round to nearest even (finite inputs)
uint16_t bf16_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP E4M3FN code of v: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no
// infinities; nearest value, ties to even; magnitudes past 448 saturate to 448.
uint8_t e4m3_code(double v) {
    const uint8_t sign = std::signbit(v) ? 0x80 : 0;
    const double a = std::fabs(v);
    if (a < 0x1p-6) {  // subnormals k * 2^-9
        const int k = (int)std::nearbyint(a * 512.0);
        return sign | (uint8_t)(k == 8 ? 0x08 : k);
    }
    int e2 = 0;
    std::frexp(a, &e2);
    int be = e2 - 1;  // a in [2^be, 2^(be+1))
    int mant = (int)std::nearbyint(std::ldexp(a, 3 - be));  // 8 .. 16
    if (mant == 16) be += 1, mant = 8;
    if (be > 8 || (be == 8 && mant > 14)) be = 8, mant = 14;
    return sign | (uint8_t)((be + 7) << 3) | (uint8_t)(mant - 8);
}

// Per-tensor E4M3: scale = amax / 448; codes of value / scale.
double e4m3_scale(uint16_t const *w, size_t n) {
    double amax = 0.0;
    for (size_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs((double)bf16_value(w[i])));
    return amax > 0.0 ? amax / 448.0 : 0.0;
}

void e4m3_encode(uint8_t *dst, uint16_t const *packed, size_t n, double scale) {
    for (size_t i = 0; i < n; ++i) dst[i] = scale > 0.0 ? e4m3_code((double)bf16_value(packed[i]) / scale) : 0;
}

// interleaved gate/up rows [2F x D]: 64b + [0,32) gate column 32b + r, 64b + [32,64) up
size_t gate_up_row(size_t col, bool up) { return 64 * (col / 32) + (up ? 32 : 0) + col % 32; }

}  // namespace

extern "C" void ube_model_init(ube_model_init_t *a) {
    if (!a) return;
    ube_outcome_t *outcome = a->outcome;
    if (a->model) *a->model = nullptr;
    ube_model_t m = nullptr;
    try {
        if (!a->model || !a->weights) throw Failure{ube_status_invalid_argument_k, "NULL model or weights"};
        ube_geometry_t g = complete_geometry(a->geometry);
        if (char const *why = check_geometry(g)) throw Failure{ube_status_unsupported_k, why};
        ube_weights_t const &w = *a->weights;
        bool text = w.embed != nullptr;
        if (text && g.vocab < 256) throw Failure{ube_status_unsupported_k, "a byte vocabulary needs >= 256 rows"};
        if (!text && !w.patch_proj) throw Failure{ube_status_invalid_argument_k, "neither embed nor patch_proj"};
        if (!text && (g.patch_side != 16 || g.channels != 3))
            throw Failure{ube_status_unsupported_k, "media frontends take 16x16 RGB patches"};
        if (!w.w_qkv || !w.w_o || !w.w_gate || !w.w_up || !w.w_down || !w.attn_norm || !w.mlp_norm || !w.final_norm ||
            !w.pool_query || !w.pool_wk || !w.pool_wv)
            throw Failure{ube_status_invalid_argument_k, "missing weights"};
        for (size_t l = 0; l < g.depth; ++l)
            if (!w.w_qkv[l] || !w.w_o[l] || !w.w_gate[l] || !w.w_up[l] || !w.w_down[l] || !w.attn_norm[l] ||
                !w.mlp_norm[l])
                throw Failure{ube_status_invalid_argument_k, "missing block weights"};
        if (g.token_width && !w.token_head) throw Failure{ube_status_invalid_argument_k, "missing token head"};
        int ndev = 0;
        if (hipGetDeviceCount(&ndev) != hipSuccess || a->device < 0 || a->device >= ndev)
            throw Failure{ube_status_device_k, "no such GPU"};
        UBE_HIP(hipSetDevice(a->device));

        const size_t D = g.hidden, F = g.ffn, H = g.heads, N = g.depth;
        const size_t KP = g.patch_side * g.patch_side * g.channels;
        // device layout
        std::vector<size_t> offs;
        size_t total = 0;
        auto take = [&](size_t bytes) {
            size_t o = total;
            total = align_up(total + bytes, 256);
            return o;
        };
        size_t o_embed = text ? take(g.vocab * D * 2) : 0;
        size_t o_patch = text ? 0 : take(D * KP * 2);
        const bool e4m3 = g.quantization == ube_scalar_e4m3_k;
        const size_t ES = e4m3 ? 1 : 2;  // bytes per block-matrix element
        std::vector<size_t> o_l(N * 6);
        for (size_t l = 0; l < N; ++l) {
            o_l[l * 6 + 0] = take(3 * D * D * ES);
            o_l[l * 6 + 1] = take(D * D * ES);
            o_l[l * 6 + 2] = take(2 * F * D * ES);
            o_l[l * 6 + 3] = take(F * D * ES);
            o_l[l * 6 + 4] = take(D * 4);
            o_l[l * 6 + 5] = take(D * 4);
        }
        size_t o_gf = take(D * 4), o_u = take(H * D * 4), o_wv = take(D * D * 2);
        size_t o_rope = take(g.context * 32 * sizeof(float2));
        size_t o_tok = g.token_width ? take(g.token_width * D * 2) : 0;

        std::vector<char> host(total);
        char *hb = host.data();
        if (text) std::memcpy(hb + o_embed, w.embed, g.vocab * D * 2);
        else transpose_into((uint16_t *)(hb + o_patch), w.patch_proj, KP, D);
        std::vector<ube_model_handle_t::Layer> scales(N);
        std::vector<uint16_t> tmp;
        // packed bf16 matrix -> its slot (as is, or as E4M3 codes of value / scale)
        auto place = [&](size_t off, std::vector<uint16_t> const &packed, double scale) {
            if (e4m3) e4m3_encode((uint8_t *)(hb + off), packed.data(), packed.size(), scale);
            else std::memcpy(hb + off, packed.data(), packed.size() * 2);
        };
        for (size_t l = 0; l < N; ++l) {
            auto &sc = scales[l];
            if (e4m3) {
                sc.s_qkv = (float)e4m3_scale(w.w_qkv[l], D * 3 * D);
                sc.s_o = (float)e4m3_scale(w.w_o[l], D * D);
                sc.s_gate = (float)e4m3_scale(w.w_gate[l], D * F);
                sc.s_up = (float)e4m3_scale(w.w_up[l], D * F);
                sc.s_down = (float)e4m3_scale(w.w_down[l], F * D);
            }
            // bf16 blocks: each RMSNorm gain folds into the projection that reads the
            // normalised rows, W'[n][k] = g[k] W[k][n] (the kernels apply 1/rms(x) to the
            // accumulator). E4M3 blocks keep W and quantise the normalised rows.
            auto fold = [&](std::vector<uint16_t> &packed, size_t K, float const *gain) {
                if (e4m3) return;
                for (size_t i = 0; i < packed.size(); ++i)
                    packed[i] = bf16_bits(bf16_value(packed[i]) * gain[i % K]);
            };
            tmp.assign(3 * D * D, 0);
            transpose_into(tmp.data(), w.w_qkv[l], D, 3 * D);
            fold(tmp, D, w.attn_norm[l]);
            place(o_l[l * 6 + 0], tmp, e4m3 ? e4m3_scale(w.w_qkv[l], D * 3 * D) : 0.0);
            tmp.assign(D * D, 0);
            transpose_into(tmp.data(), w.w_o[l], D, D);
            place(o_l[l * 6 + 1], tmp, e4m3 ? e4m3_scale(w.w_o[l], D * D) : 0.0);
            // gate/up interleaved in blocks of 32 output columns; E4M3 keeps one scale per tensor
            tmp.assign(2 * F * D, 0);
            for (size_t col = 0; col < F; ++col)
                for (size_t k = 0; k < D; ++k) {
                    tmp[gate_up_row(col, false) * D + k] = w.w_gate[l][k * F + col];
                    tmp[gate_up_row(col, true) * D + k] = w.w_up[l][k * F + col];
                }
            fold(tmp, D, w.mlp_norm[l]);
            if (e4m3) {
                const double sg = e4m3_scale(w.w_gate[l], D * F), su = e4m3_scale(w.w_up[l], D * F);
                uint8_t *dst = (uint8_t *)(hb + o_l[l * 6 + 2]);
                for (size_t r = 0; r < 2 * F; ++r) {
                    const double sr = ((r / 32) & 1) ? su : sg;
                    e4m3_encode(dst + r * D, tmp.data() + r * D, D, sr);
                }
            } else {
                place(o_l[l * 6 + 2], tmp, 0.0);
            }
            tmp.assign(F * D, 0);
            transpose_into(tmp.data(), w.w_down[l], F, D);
            place(o_l[l * 6 + 3], tmp, e4m3 ? e4m3_scale(w.w_down[l], F * D) : 0.0);
            std::memcpy(hb + o_l[l * 6 + 4], w.attn_norm[l], D * 4);
            std::memcpy(hb + o_l[l * 6 + 5], w.mlp_norm[l], D * 4);
        }
        std::memcpy(hb + o_gf, w.final_norm, D * 4);
        // pool keys folded into the query: u_h = W_k[:, head h] q_h / sqrt(64)
        float *u = (float *)(hb + o_u);
        for (size_t h = 0; h < H; ++h)
            for (size_t f = 0; f < D; ++f) {
                double acc = 0.0;
                for (size_t e = 0; e < 64; ++e)
                    acc += (double)bf16_value(w.pool_wk[f * D + h * 64 + e]) * (double)bf16_value(w.pool_query[h * 64 + e]);
                u[h * D + f] = (float)(acc / 8.0);
            }
        std::memcpy(hb + o_wv, w.pool_wv, D * D * 2);
        if (g.token_width) transpose_into((uint16_t *)(hb + o_tok), w.token_head, D, g.token_width);
        // rotary table: (cos, sin) of p * base^(-2j/64), double on the host
        float2 *rope = (float2 *)(hb + o_rope);
        for (size_t p = 0; p < g.context; ++p)
            for (size_t j = 0; j < 32; ++j) {
                double theta = std::pow((double)g.rope_base, -2.0 * (double)j / 64.0);
                double phi = (double)p * theta;
                rope[p * 32 + j] = float2{(float)std::cos(phi), (float)std::sin(phi)};
            }

        m = new ube_model_handle_t();
        m->device = a->device;
        m->g = g;
        m->text = text;
        m->bytes = total;
        UBE_HIP(hipMalloc((void **)&m->mem, total));
        UBE_HIP(hipMemcpy(m->mem, hb, total, hipMemcpyHostToDevice));
        char *db = m->mem;
        m->embed = text ? (uint16_t *)(db + o_embed) : nullptr;
        m->patch_t = text ? nullptr : (uint16_t *)(db + o_patch);
        m->layers.resize(N);
        m->e4m3 = e4m3;
        for (size_t l = 0; l < N; ++l) {
            m->layers[l] = scales[l];
            m->layers[l].wqkv = (uint16_t *)(db + o_l[l * 6 + 0]);
            m->layers[l].wo = (uint16_t *)(db + o_l[l * 6 + 1]);
            m->layers[l].wgu = (uint16_t *)(db + o_l[l * 6 + 2]);
            m->layers[l].wd = (uint16_t *)(db + o_l[l * 6 + 3]);
            m->layers[l].g1 = (float *)(db + o_l[l * 6 + 4]);
            m->layers[l].g2 = (float *)(db + o_l[l * 6 + 5]);
        }
        m->gf = (float *)(db + o_gf);
        m->u = (float *)(db + o_u);
        m->wv = (uint16_t *)(db + o_wv);
        m->rope = (float2 *)(db + o_rope);
        m->tok = g.token_width ? (uint16_t *)(db + o_tok) : nullptr;
        const int pairs = 32, axes = (int)g.rope_axes, base = pairs / axes, rem = pairs % axes;
        m->sec0 = base + (0 < rem ? 1 : 0);
        m->sec1 = axes >= 2 ? base + (1 < rem ? 1 : 0) : 0;
        *a->model = m;
        set_outcome(outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        if (m) {
            if (m->mem) (void)hipFree(m->mem);
            delete m;
        }
        set_outcome(outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        if (m) {
            if (m->mem) (void)hipFree(m->mem);
            delete m;
        }
        set_outcome(outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

extern "C" void ube_model_describe(ube_model_describe_t *a) {
    if (!a) return;
    if (!a->model || !a->description) {
        set_outcome(a->outcome, ube_status_invalid_argument_k, "NULL model or description");
        return;
    }
    ube_model_t m = a->model;
    ube_model_description_t &d = *a->description;
    d.dimensions = m->g.hidden;
    d.context = m->g.context;
    d.depth = m->g.depth;
    d.heads = m->g.heads;
    d.ffn = m->g.ffn;
    d.rope_axes = m->g.rope_axes;
    d.quantization = m->g.quantization;
    d.memory_usage = m->bytes;
    d.device = m->device;
    d.token_width = m->g.token_width;
    set_outcome(a->outcome, ube_status_success_k, nullptr);
}

extern "C" void ube_model_free(ube_model_t m) {
    if (!m) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(m->device);
    (void)hipFree(m->mem);
    (void)hipSetDevice(prev);
    delete m;
}

// ===================================================================== arena

struct ube_arena_handle_t {
    int device = 0;
    std::atomic<int> busy{0};
    char *dev = nullptr;
    size_t cap = 0;
    size_t limit = 0;  // device bytes the arena may hold (0: no limit)
    char *pinned = nullptr;
    size_t pinned_cap = 0;
    hipEvent_t staged = nullptr;  // recorded after the last copy out of `pinned`
    bool staged_pending = false;
};

extern "C" void ube_arena_init(ube_arena_init_t *a) {
    if (!a) return;
    if (!a->arena) {
        set_outcome(a->outcome, ube_status_invalid_argument_k, "NULL arena output");
        return;
    }
    *a->arena = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || a->device < 0 || a->device >= ndev) {
        set_outcome(a->outcome, ube_status_device_k, "no such GPU");
        return;
    }
    ube_arena_t ar = new (std::nothrow) ube_arena_handle_t();
    if (!ar) {
        set_outcome(a->outcome, ube_status_out_of_memory_k, "host out of memory");
        return;
    }
    ar->device = a->device;
    ar->limit = a->capacity_limit;
    *a->arena = ar;
    set_outcome(a->outcome, ube_status_success_k, nullptr);
}

extern "C" void ube_arena_free(ube_arena_t ar) {
    if (!ar) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(ar->device);
    (void)hipDeviceSynchronize();
    if (ar->dev) (void)hipFree(ar->dev);
    if (ar->pinned) (void)hipHostFree(ar->pinned);
    if (ar->staged) (void)hipEventDestroy(ar->staged);
    (void)hipSetDevice(prev);
    delete ar;
}

extern "C" size_t ube_arena_capacity(ube_arena_t ar) { return ar ? ar->cap : 0; }

namespace {

// Grows the arena to hold `total` bytes (whole MiB), only when outgrown; the old contents are not kept.
// Beyond the arena's capacity limit the call fails out_of_memory and the arena keeps what it holds.
void arena_reserve(ube_arena_t ar, size_t total, hipStream_t st, bool clear) {
    if (total <= ar->cap) return;
    const size_t want = align_up(total, (size_t)1 << 20);
    if (ar->limit && want > ar->limit)
        throw Failure{ube_status_out_of_memory_k, "the call needs more device memory than the arena's capacity limit"};
    UBE_HIP(hipStreamSynchronize(st));
    if (ar->dev) UBE_HIP(hipFree(ar->dev));
    ar->dev = nullptr;
    ar->cap = 0;
    UBE_HIP(hipMalloc((void **)&ar->dev, want));
    ar->cap = want;
    if (clear) UBE_HIP(hipMemsetAsync(ar->dev, 0, want, st));
}

}  // namespace

// ===================================================================== plan

extern "C" ube_status_t ube_tape_plan(size_t const *offsets, size_t count, size_t context, uint32_t *lengths,
                                      uint32_t *cu, ube_encode_stats_t *stats) {
    if (!offsets || !cu || (count && !lengths)) return ube_status_invalid_argument_k;
    size_t truncated = 0, tokens = 0;
    cu[0] = 0;
    for (size_t i = 0; i < count; ++i) {
        if (offsets[i + 1] < offsets[i]) return ube_status_invalid_argument_k;
        size_t len = offsets[i + 1] - offsets[i];
        size_t kept = len > context ? context : len;
        truncated += len > context;
        lengths[i] = (uint32_t)kept;
        tokens += kept;
        if (tokens > 0x7fffffffull - 4096) return ube_status_invalid_argument_k;
        cu[i + 1] = (uint32_t)tokens;
    }
    if (stats) stats->truncated = truncated, stats->tokens = tokens;
    return ube_status_success_k;
}

namespace {

struct Plan {
    size_t count = 0, T = 0, truncated = 0;
    std::vector<int> cu;            // count + 1
    std::vector<int64_t> src;       // count: byte offset of each item in the device input
    std::vector<int2> tiles;        // (item, first token) per 256-token tile, in item order
    std::vector<int2> atiles;       // the same tiles in the attention's launch order (longest items first)
    std::vector<int> itile;         // count + 1: first tile of each item
    std::vector<MediaItem> media;   // media items
    size_t input_lo = 0, input_hi = 0;  // tape data range the items read
};

constexpr size_t kLongestFirstTiles = 1024;

void make_tiles(Plan &p) {
    p.tiles.clear();
    p.itile.assign(p.count + 1, 0);
    for (size_t i = 0; i < p.count; ++i) {
        p.itile[i] = (int)p.tiles.size();
        for (int t = p.cu[i]; t < p.cu[i + 1]; t += kTileTokens) p.tiles.push_back(int2{(int)i, t});
    }
    p.itile[p.count] = (int)p.tiles.size();
    // An attention workgroup's work grows with its item's length (all of the item's keys). When the
    // attention grid is only a few rounds of workgroups (up to kLongestFirstTiles tiles per head), the
    // round in which the longest items' tiles start decides the end, so those tiles go first and the
    // short ones fill the last round (longest-first scheduling; each XCD runs a contiguous range of the
    // grid, one head's tiles in this order when there are 8 heads). Larger grids keep item order, whose
    // neighbouring workgroups read neighbouring rows (ragged 64-item batch: attention 80 -> 72 us; a
    // 4096-segment batch: 1.58 ms in item order, 1.60 sorted). Equal lengths keep item order either
    // way, and results do not depend on the order.
    p.atiles = p.tiles;
    if (p.tiles.size() <= kLongestFirstTiles)
        std::stable_sort(p.atiles.begin(), p.atiles.end(), [&](int2 a, int2 b) {
            return p.cu[a.x + 1] - p.cu[a.x] > p.cu[b.x + 1] - p.cu[b.x];
        });
}

// Device regions of one call.
struct Layout {
    size_t Tpad = 0;
    size_t out, cu, offs, src, tiles, atiles, itile, media, input, x, h, a, qk, vt, o, xf, s, pos, patches, q8, qs,
        ss, st, tvf, tv, zp, zs, total;
};

// Per-token surfaces of one call: fp32 states (bf16 states are the final-norm
// rows themselves), token vectors.
struct TokenOutputs {
    bool states_f32 = false, vectors = false;
    size_t width = 0, vector_bytes = 2;
};

Layout carve(ube_geometry_t const &g, Plan const &p, bool media, size_t input_bytes, bool e4m3,
             TokenOutputs const &tok) {
    Layout L{};
    const size_t D = g.hidden, F = g.ffn, H = g.heads;
    L.Tpad = align_up(p.T, 256) + kRowPad;
    size_t total = 0;
    auto take = [&](size_t bytes) {
        size_t o = total;
        total = align_up(total + bytes, 256);
        return o;
    };
    L.out = take(std::max<size_t>(p.count, 1) * D * 4);
    L.cu = take((p.count + 1) * 4);
    L.offs = take((p.count + 1) * 8);  // the token offsets as size_t, for rows tapes
    L.src = take(std::max<size_t>(p.count, 1) * 8);
    L.tiles = take(std::max<size_t>(p.tiles.size(), 1) * 8);
    L.atiles = take(std::max<size_t>(p.tiles.size(), 1) * 8);
    L.itile = take((p.count + 1) * 4);
    L.media = take(media ? std::max<size_t>(p.count, 1) * sizeof(MediaItem) : 0);
    L.input = take(input_bytes);
    L.x = take(L.Tpad * D * 4);
    L.h = take(L.Tpad * D * 2);
    L.a = take(L.Tpad * F * 2);
    L.qk = take(L.Tpad * 2 * D * 2);
    L.vt = take(D * L.Tpad * 2);
    L.o = take(L.Tpad * D * 2);
    L.xf = take(L.Tpad * D * 2);
    L.s = take(L.Tpad * H * 4);
    L.pos = take(L.Tpad * 4 * 2);
    L.patches = take(media ? L.Tpad * 768 * 2 : 0);
    L.q8 = take(e4m3 ? L.Tpad * std::max(D, F) : 0);  // E4M3 GEMM input rows
    L.qs = take(e4m3 ? L.Tpad * 4 : 0);               // their per-row scales
    L.ss = take(L.Tpad * kSsParts * 4);               // partial sums of squares of x
    L.st = take(tok.states_f32 ? L.Tpad * D * 4 : 0);
    L.tvf = take(tok.vectors ? L.Tpad * tok.width * 4 : 0);  // token head output before normalisation
    L.tv = take(tok.vectors ? L.Tpad * tok.width * tok.vector_bytes : 0);
    L.zp = take(pool_partial_bytes((int)p.tiles.size(), (int)D, (int)H));  // pool: per-tile partial sums
    L.zs = take(pool_stats_bytes((int)p.tiles.size(), (int)H));
    L.total = total;
    return L;
}

bool pointer_on_device(void const *ptr, int device) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeDevice && attr.device == device;
}

// Guards an arena for one call.
struct ArenaLease {
    ube_arena_t ar;
    bool held = false;
    explicit ArenaLease(ube_arena_t a) : ar(a) {
        int expected = 0;
        held = ar->busy.compare_exchange_strong(expected, 1);
    }
    ~ArenaLease() {
        if (held) ar->busy.store(0);
    }
};

// Where a training forward leaves the activations its backward reads (device memory outside the arena):
// every block's fp32 input (and the final norm's, at block N) and the final-norm rows and pool scores;
// unless the backward recomputes them (x1 and qk NULL), also the fp32 rows after each block's attention
// half and each block's rotated q|k rows, feature-major v, attention output and softmax log2 denominators.
struct Keep {
    float *x;         // [(N + 1) x T x D]
    float *x1;        // [N x T x D] or NULL
    uint16_t *qk;     // [N][Tpad x 2D] or NULL (then vt, o, lse, gu unused)
    uint16_t *vt;     // [N][D x ldvt]
    uint16_t *o;      // [N][Tpad x D]
    float *lse;       // [N][H x ldl]
    uint16_t *gu;     // [N][Tpad x 2F] gate/up pre-activations (interleaved as the packed weights) or NULL
    uint16_t *xf;     // [Tpad x D]
    float *s;         // [Tpad x H]
    size_t Tpad, ldvt, ldl;
};

struct EncodeRequest {
    ube_model_t model;
    ube_arena_t arena;
    hipStream_t stream;
    int completion;
    ube_scalar_t outputs_scalar;
    ube_rows_view_t *embeddings;
    ube_encode_stats_t *stats;
    float *trace;
    void const *data;      // tape data
    size_t const *offsets; // host
    size_t count;
    unsigned outputs;
    ube_rows_tape_view_t *states;
    ube_rows_tape_view_t *token_vectors;
    Layout *layout = nullptr;  // when set, receives the call's arena layout (the trainer reads cu, tiles)
    Keep const *keep = nullptr;  // training forward: where the backward's activations go
};


bool wants(unsigned outputs, ube_outputs_t o) { return (outputs ? outputs : ube_outputs_embeddings_k) & o; }

// Runs the whole encode for a prepared plan. `media` selects the patch frontend.
void run_encode(EncodeRequest const &r, Plan &p, bool media) {
    ube_model_t m = r.model;
    ube_arena_t ar = r.arena;
    ube_geometry_t const &g = m->g;
    const int D = (int)g.hidden, F = (int)g.ffn, H = (int)g.heads;
    const float eps = g.rms_epsilon;
    hipStream_t st = r.stream;

    // tape data: in place when it already lives on this GPU, else staged through the arena
    const bool on_device = p.input_hi > p.input_lo ? pointer_on_device(r.data, m->device) : true;
    const size_t input_bytes = on_device ? 0 : p.input_hi - p.input_lo;
    if (on_device && ar->dev && p.input_hi > p.input_lo) {
        char const *lo = (char const *)r.data + p.input_lo, *hi = (char const *)r.data + p.input_hi;
        if (hi > ar->dev && lo < ar->dev + ar->cap)
            throw Failure{ube_status_invalid_argument_k, "inputs lie inside the arena"};
    }
    const bool bf16_out = r.outputs_scalar == ube_scalar_bf16_k;
    TokenOutputs tok;
    tok.states_f32 = wants(r.outputs, ube_outputs_states_k) && !bf16_out;
    tok.vectors = wants(r.outputs, ube_outputs_token_vectors_k);
    tok.width = g.token_width;
    tok.vector_bytes = bf16_out ? 2 : 4;
    Layout L = carve(g, p, media, input_bytes, m->e4m3, tok);
    if (r.layout) *r.layout = L;

    // grow the arena (only when outgrown)
    arena_reserve(ar, L.total, st, true);
    char *db = ar->dev;

    // host staging: cu, src, tiles, media items (+ tape bytes when host-resident)
    const size_t meta_bytes = L.input - L.cu;
    const size_t stage_bytes = meta_bytes + input_bytes;
    if (ar->staged_pending) {
        UBE_HIP(hipEventSynchronize(ar->staged));
        ar->staged_pending = false;
    }
    if (stage_bytes > ar->pinned_cap) {
        if (ar->pinned) UBE_HIP(hipHostFree(ar->pinned));
        ar->pinned = nullptr;
        ar->pinned_cap = 0;
        size_t want = align_up(stage_bytes, (size_t)1 << 16);
        UBE_HIP(hipHostMalloc((void **)&ar->pinned, want, 0));
        ar->pinned_cap = want;
    }
    if (!ar->staged) UBE_HIP(hipEventCreateWithFlags(&ar->staged, hipEventDisableTiming));
    char *hp = ar->pinned;
    std::memset(hp, 0, meta_bytes);
    std::memcpy(hp + (L.cu - L.cu), p.cu.data(), p.cu.size() * 4);
    for (size_t i = 0; i <= p.count; ++i) ((uint64_t *)(hp + (L.offs - L.cu)))[i] = (uint64_t)p.cu[i];
    for (size_t i = 0; i < p.count; ++i)
        ((int64_t *)(hp + (L.src - L.cu)))[i] = p.src[i] - (on_device ? 0 : (int64_t)p.input_lo);
    if (!p.tiles.empty()) std::memcpy(hp + (L.tiles - L.cu), p.tiles.data(), p.tiles.size() * 8);
    if (!p.atiles.empty()) std::memcpy(hp + (L.atiles - L.cu), p.atiles.data(), p.atiles.size() * 8);
    std::memcpy(hp + (L.itile - L.cu), p.itile.data(), p.itile.size() * 4);
    if (media && p.count) {
        std::vector<MediaItem> items = p.media;
        for (auto &it : items) it.pixel_offset -= on_device ? 0 : (int64_t)p.input_lo;
        std::memcpy(hp + (L.media - L.cu), items.data(), items.size() * sizeof(MediaItem));
    }
    if (input_bytes) std::memcpy(hp + meta_bytes, (char const *)r.data + p.input_lo, input_bytes);
    UBE_HIP(hipMemcpyAsync(db + L.cu, hp, stage_bytes, hipMemcpyHostToDevice, st));
    UBE_HIP(hipEventRecord(ar->staged, st));
    ar->staged_pending = true;

    const uint8_t *input = on_device ? (const uint8_t *)r.data : (const uint8_t *)(db + L.input);
    const int *cu = (const int *)(db + L.cu);
    const int64_t *src = (const int64_t *)(db + L.src);
    const int2 *tiles = (const int2 *)(db + L.tiles), *atiles = (const int2 *)(db + L.atiles);
    const int ntiles = (int)p.tiles.size();
    float *x = (float *)(db + L.x);
    uint16_t *h = (uint16_t *)(db + L.h), *act = (uint16_t *)(db + L.a), *qk = (uint16_t *)(db + L.qk);
    uint16_t *vt = (uint16_t *)(db + L.vt), *o = (uint16_t *)(db + L.o), *xf = (uint16_t *)(db + L.xf);
    float *s = (float *)(db + L.s);
    int16_t *pos = (int16_t *)(db + L.pos);
    float *ssq = (float *)(db + L.ss);
    const int T = (int)p.T, ldvt = (int)L.Tpad;

    if (T > 0) {
        // the residual stream: in place in the arena, or (training forward) block l's fp32 input kept at
        // keep->x + l T D and the rows after its attention half at keep->x1 + l T D (the arena's x when
        // those are recomputed), every residual product writing out of place
        Keep const *kp = r.keep;
        const size_t TD = (size_t)T * D;
        auto xin = [&](size_t l) { return kp ? kp->x + l * TD : x; };
        auto xmid = [&](size_t l) { return kp && kp->x1 ? kp->x1 + l * TD : x; };
        // keys past the last token are masked; their values must still be finite (p = 0 times v)
        UBE_HIP(hipMemset2DAsync(vt + T, (size_t)ldvt * 2, 0, 64 * 2, (size_t)D, st));
        // ---- frontend
        if (!media) {
            timed(ube_kernel_gather_k, st, [&] {
                return launch_gather_text(input, src, cu, tiles, ntiles, m->embed, xin(0), h, ssq, pos, D, st);
            });
        } else {
            uint16_t *patches = (uint16_t *)(db + L.patches);
            timed(ube_kernel_patchify_k, st, [&] {
                return launch_patchify(input, (const MediaItem *)(db + L.media), cu, tiles, ntiles, patches, pos,
                                       (int)g.rope_axes, st);
            });
            GemmArgs ga{};
            ga.w = m->patch_t, ga.x = patches, ga.M = T, ga.N = D, ga.K = 768;
            ga.out_f32 = xin(0), ga.ld_f32 = D, ga.scale = 1.0f / 255.0f;
            ga.out_bf16 = h, ga.ld_out = D, ga.ss_out = ssq;
            timed(ube_kernel_gemm_patch_k, st, [&] { return launch_gemm(kEpiPatch, ga, st); });
        }
        if (r.trace) UBE_HIP(hipMemcpyAsync(r.trace, xin(0), TD * 4, hipMemcpyDeviceToDevice, st));
        // ---- blocks
        uint8_t *q8 = (uint8_t *)(db + L.q8);
        float *qs = (float *)(db + L.qs);
        // one projection: bf16 operands, or E4M3 rows (codes + per-row scales) against E4M3 weights
        auto project = [&](ube_kernel_t kind, int epi, GemmArgs ga, float w_scale, float w_scale2) {
            if (m->e4m3) {
                ga.x = (const uint16_t *)q8, ga.x_scale = qs, ga.w_scale = w_scale, ga.w_scale2 = w_scale2;
                timed(kind, st, [&] { return launch_gemm_e4m3(epi, ga, st); });
            } else {
                timed(kind, st, [&] { return launch_gemm(epi, ga, st); });
            }
        };
        // RMSNorm into the next projection's input (bf16 h, or E4M3 rows)
        auto norm = [&](const float *xr, const float *gain) {
            if (m->e4m3)
                timed(ube_kernel_rmsnorm_k, st, [&] { return launch_rmsnorm_e4m3(xr, gain, q8, qs, T, D, eps, st); });
            else
                timed(ube_kernel_rmsnorm_k, st, [&] { return launch_rmsnorm(xr, gain, h, T, D, eps, st); });
        };
        auto quantize = [&](const uint16_t *rows, int width) {
            timed(ube_kernel_quantize_k, st, [&] { return launch_quantize_rows(rows, q8, qs, T, width, st); });
        };
        // bf16: the normalisation of the rows a projection reads is folded into it
        // (x's bf16 copy h in, gain in the weights, 1/rms from the partial sums)
        auto folded_norm = [&](GemmArgs &ga) {
            // producers of x (residual and patch GEMMs, N = D) write one partial per
            // 256 features from the 256-wide kernel, else one per 64 (gather: part 0)
            if (!m->e4m3) ga.ss_in = ssq, ga.ss_parts = D % 256 == 0 ? D / 256 : D / 64, ga.eps = eps;
        };
        auto residual_out = [&](GemmArgs &ga) {
            if (!m->e4m3) ga.out_bf16 = h, ga.ld_out = D, ga.ss_out = ssq;
        };
        for (size_t l = 0; l < g.depth; ++l) {
            auto const &Wl = m->layers[l];
            // this block's q|k, v and attention rows: the arena's scratch, or the training forward's own
            uint16_t *qk_l = qk, *vt_l = vt, *o_l = o;
            int ldvt_l = ldvt;
            float *lse_l = nullptr;
            float *x_l = xin(l), *x1_l = xmid(l), *x_next = xin(l + 1);
            if (kp && kp->qk) {
                qk_l = kp->qk + l * kp->Tpad * 2 * D, vt_l = kp->vt + l * D * kp->ldvt, o_l = kp->o + l * kp->Tpad * D;
                ldvt_l = (int)kp->ldvt, lse_l = kp->lse + l * H * kp->ldl;
                UBE_HIP(hipMemset2DAsync(vt_l + T, kp->ldvt * 2, 0, 64 * 2, (size_t)D, st));
            }
            if (m->e4m3) norm(x_l, Wl.g1);
            GemmArgs qa{};
            qa.w = Wl.wqkv, qa.x = h, qa.M = T, qa.N = 3 * D, qa.K = D;
            folded_norm(qa);
            qa.out_bf16 = qk_l, qa.ld_out = 2 * D, qa.vt = vt_l, qa.ld_vt = ldvt_l, qa.pos = pos, qa.rope = m->rope;
            qa.D = D, qa.sec0 = m->sec0, qa.sec1 = m->sec1;
            project(ube_kernel_gemm_qkv_k, kEpiQkv, qa, Wl.s_qkv, 0.f);
            timed(ube_kernel_attention_k, st, [&] {
                return launch_attention(qk_l, qk_l + D, 2 * D, vt_l, ldvt_l, o_l, D, cu, atiles, ntiles, H, st, lse_l,
                                        lse_l ? (int)kp->ldl : 0);
            });
            if (m->e4m3) quantize(o_l, D);
            GemmArgs oa{};
            oa.w = Wl.wo, oa.x = o_l, oa.M = T, oa.N = D, oa.K = D, oa.out_f32 = x1_l, oa.ld_f32 = D;
            oa.res_in = x1_l == x_l ? nullptr : x_l;
            residual_out(oa);
            project(ube_kernel_gemm_out_k, kEpiResid, oa, Wl.s_o, 0.f);
            if (m->e4m3) norm(x1_l, Wl.g2);
            GemmArgs ua{};
            ua.w = Wl.wgu, ua.x = h, ua.M = T, ua.N = 2 * F, ua.K = D, ua.out_bf16 = act, ua.ld_out = F;
            if (kp && kp->gu) ua.gu_out = kp->gu + l * kp->Tpad * 2 * F, ua.ld_gu = 2 * F;
            folded_norm(ua);
            project(ube_kernel_gemm_gate_up_k, kEpiSwiglu, ua, Wl.s_gate, Wl.s_up);
            if (m->e4m3) quantize(act, F);
            GemmArgs da{};
            da.w = Wl.wd, da.x = act, da.M = T, da.N = D, da.K = F, da.out_f32 = x_next, da.ld_f32 = D;
            da.res_in = x_next == x1_l ? nullptr : x1_l;
            residual_out(da);
            project(ube_kernel_gemm_down_k, kEpiResid, da, Wl.s_down, 0.f);
            if (r.trace) UBE_HIP(hipMemcpyAsync(r.trace + (l + 1) * TD, x_next, TD * 4, hipMemcpyDeviceToDevice, st));
        }
        if (kp) xf = kp->xf, s = kp->s;
        float *states = tok.states_f32 ? (float *)(db + L.st) : nullptr;
        timed(ube_kernel_final_norm_k, st,
              [&] { return launch_final_norm_scores(xin(g.depth), m->gf, m->u, xf, s, states, T, D, H, eps, st); });
        if (tok.vectors) {
            // token head (bf16 operands, fp32 rows), then unit rows
            GemmArgs ta{};
            ta.w = m->tok, ta.x = xf, ta.M = T, ta.N = (int)tok.width, ta.K = D;
            ta.out_f32 = (float *)(db + L.tvf), ta.ld_f32 = (int)tok.width, ta.scale = 1.0f;
            UBE_HIP(launch_gemm(kEpiPatch, ta, st));
            UBE_HIP(launch_unit_rows((const float *)(db + L.tvf), db + L.tv, bf16_out ? 1 : 0, T, (int)tok.width, st));
        }
    }
    const size_t row_bytes = (size_t)D * (bf16_out ? 2 : 4);
    const bool embeddings = wants(r.outputs, ube_outputs_embeddings_k);
    if (p.count && embeddings) {
        timed(ube_kernel_pool_k, st, [&] {
            return launch_pool(xf, s, cu, tiles, ntiles, (const int *)(db + L.itile), (int)p.count, m->wv, db + L.out,
                               bf16_out ? 1 : 0, row_bytes, D, H, (float *)(db + L.zp), (float2 *)(db + L.zs), st);
        });
    }
    if (r.completion == 0) UBE_HIP(hipStreamSynchronize(st));
    UBE_HIP(hipGetLastError());
    const ube_scalar_t scalar = bf16_out ? ube_scalar_bf16_k : ube_scalar_f32_k;
    if (r.embeddings) {
        *r.embeddings = embeddings ? ube_rows_view_t{db + L.out, p.count, (size_t)D, row_bytes, scalar}
                                   : ube_rows_view_t{nullptr, 0, 0, 0, ube_scalar_unknown_k};
    }
    size_t const *offs = (size_t const *)(db + L.offs);
    if (r.states) {
        *r.states = wants(r.outputs, ube_outputs_states_k)
                        ? ube_rows_tape_view_t{bf16_out ? (void *)(db + L.xf) : (void *)(db + L.st), offs, p.count,
                                               p.T, (size_t)D, row_bytes, scalar}
                        : ube_rows_tape_view_t{nullptr, nullptr, 0, 0, 0, 0, ube_scalar_unknown_k};
    }
    if (r.token_vectors) {
        *r.token_vectors = tok.vectors ? ube_rows_tape_view_t{db + L.tv, offs, p.count, p.T, tok.width,
                                                              tok.width * tok.vector_bytes, scalar}
                                       : ube_rows_tape_view_t{nullptr, nullptr, 0, 0, 0, 0, ube_scalar_unknown_k};
    }
    if (r.stats) r.stats->truncated = p.truncated, r.stats->tokens = p.T;
}

void check_common(ube_model_t model, ube_arena_t arena, ube_rows_view_t *embeddings, ube_scalar_t outputs_scalar,
                  unsigned outputs, ube_rows_tape_view_t *states, ube_rows_tape_view_t *token_vectors) {
    if (outputs & ~7u) throw Failure{ube_status_invalid_argument_k, "unknown output surface"};
    if (!embeddings && wants(outputs, ube_outputs_embeddings_k))
        throw Failure{ube_status_invalid_argument_k, "NULL embeddings output"};
    if (!states && wants(outputs, ube_outputs_states_k))
        throw Failure{ube_status_invalid_argument_k, "NULL states output"};
    if (!token_vectors && wants(outputs, ube_outputs_token_vectors_k))
        throw Failure{ube_status_invalid_argument_k, "NULL token vectors output"};
    if (!model) throw Failure{ube_status_invalid_argument_k, "NULL model"};
    if (!arena) throw Failure{ube_status_invalid_argument_k, "NULL arena"};
    if (outputs_scalar != ube_scalar_unknown_k && outputs_scalar != ube_scalar_f32_k &&
        outputs_scalar != ube_scalar_bf16_k)
        throw Failure{ube_status_invalid_argument_k, "outputs_scalar must be f32 or bf16"};
    if (arena->device != model->device) throw Failure{ube_status_device_k, "arena and model on different GPUs"};
    if (wants(outputs, ube_outputs_token_vectors_k) && !model->g.token_width)
        throw Failure{ube_status_unsupported_k, "the model has no token head"};
}

template <typename Body>
void guarded(ube_outcome_t *outcome, ube_rows_view_t *embeddings, ube_rows_tape_view_t *states,
             ube_rows_tape_view_t *token_vectors, ube_arena_t arena, Body body) {
    auto clear = [&] {
        if (embeddings) *embeddings = ube_rows_view_t{nullptr, 0, 0, 0, ube_scalar_unknown_k};
        if (states) *states = ube_rows_tape_view_t{nullptr, nullptr, 0, 0, 0, 0, ube_scalar_unknown_k};
        if (token_vectors) *token_vectors = ube_rows_tape_view_t{nullptr, nullptr, 0, 0, 0, 0, ube_scalar_unknown_k};
    };
    clear();
    try {
        if (!arena) throw Failure{ube_status_invalid_argument_k, "NULL arena"};
        ArenaLease lease(arena);
        if (!lease.held) throw Failure{ube_status_contended_k, "the arena is serving another call"};
        UBE_HIP(hipSetDevice(arena->device));
        body();
        set_outcome(outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        clear();
        set_outcome(outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        clear();
        set_outcome(outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

}  // namespace

namespace {

// The plan of a byte tape: kept lengths, token prefix sums, item sources and tiles.
Plan text_plan(ube_model_t model, ube_tape_view_t const &texts) {
    const size_t count = texts.count;
    if (count && (!texts.offsets || !texts.data)) throw Failure{ube_status_invalid_argument_k, "NULL tape"};
    Plan p;
    p.count = count;
    p.cu.resize(count + 1);
    std::vector<uint32_t> lengths(count), cu(count + 1);
    ube_encode_stats_t st{};
    static const size_t zero = 0;
    if (ube_tape_plan(count ? texts.offsets : &zero, count, model->g.context, lengths.data(), cu.data(), &st) !=
        ube_status_success_k)
        throw Failure{ube_status_invalid_argument_k, "tape offsets decrease"};
    p.T = st.tokens;
    p.truncated = st.truncated;
    p.src.resize(count);
    for (size_t i = 0; i <= count; ++i) p.cu[i] = (int)cu[i];
    for (size_t i = 0; i < count; ++i) p.src[i] = (int64_t)texts.offsets[i];
    if (count) {
        p.input_lo = texts.offsets[0];
        p.input_hi = texts.offsets[0];
        for (size_t i = 0; i < count; ++i) p.input_hi = std::max(p.input_hi, texts.offsets[i] + lengths[i]);
    }
    make_tiles(p);
    return p;
}

}  // namespace

extern "C" void ube_text_encode(ube_text_encode_t *a) {
    if (!a) return;
    guarded(a->outcome, a->embeddings, a->states, a->token_vectors, a->arena, [&] {
        check_common(a->model, a->arena, a->embeddings, a->outputs_scalar, a->outputs, a->states, a->token_vectors);
        if (!a->model->text) throw Failure{ube_status_unsupported_k, "the model has no byte frontend"};
        const size_t count = a->texts.count;
        Plan p = text_plan(a->model, a->texts);
        EncodeRequest r{a->model, a->arena, (hipStream_t)a->stream, a->completion, a->outputs_scalar,
                        a->embeddings, a->stats, a->trace_residual, a->texts.data, a->texts.offsets, count,
                        a->outputs, a->states, a->token_vectors};
        run_encode(r, p, false);
    });
}

namespace {

void media_encode(ube_model_t model, ube_arena_t arena, void *stream, int completion, ube_tape_view_t tape,
                  size_t const *frame_counts, size_t const *heights, size_t const *widths, ube_scalar_t scalar,
                  ube_rows_view_t *embeddings, ube_encode_stats_t *stats, float *trace, int axes_expected,
                  unsigned outputs, ube_rows_tape_view_t *states, ube_rows_tape_view_t *token_vectors) {
    check_common(model, arena, embeddings, scalar, outputs, states, token_vectors);
    if (model->text) throw Failure{ube_status_unsupported_k, "the model has no patch frontend"};
    if ((int)model->g.rope_axes != axes_expected)
        throw Failure{ube_status_unsupported_k, "the model's rotary axes do not fit this input"};
    const size_t count = tape.count;
    if (count && (!tape.offsets || !tape.data || !heights || !widths))
        throw Failure{ube_status_invalid_argument_k, "NULL tape or sizes"};
    const size_t ps = model->g.patch_side, ch = model->g.channels;
    Plan p;
    p.count = count;
    p.cu.assign(count + 1, 0);
    p.src.assign(count, 0);
    p.media.resize(count);
    size_t T = 0;
    for (size_t i = 0; i < count; ++i) {
        if (tape.offsets[i + 1] < tape.offsets[i]) throw Failure{ube_status_invalid_argument_k, "tape offsets decrease"};
        const size_t Hh = heights[i], Ww = widths[i], Fr = frame_counts ? frame_counts[i] : 1;
        if (Hh % ps || Ww % ps || !Hh || !Ww || !Fr)
            throw Failure{ube_status_shape_mismatch_k, "a side is not a positive multiple of the patch side"};
        if (tape.offsets[i + 1] - tape.offsets[i] != Fr * Hh * Ww * ch)
            throw Failure{ube_status_shape_mismatch_k, "item bytes differ from frames x height x width x channels"};
        const size_t n = Fr * (Hh / ps) * (Ww / ps);
        if (n > model->g.context) throw Failure{ube_status_shape_mismatch_k, "patch count exceeds the context"};
        p.media[i] = MediaItem{(int64_t)tape.offsets[i], (int)Fr, (int)(Hh / ps), (int)(Ww / ps), (int)Ww};
        T += n;
        if (T > 0x7fffffffull - 4096) throw Failure{ube_status_invalid_argument_k, "too many tokens"};
        p.cu[i + 1] = (int)T;
        p.src[i] = (int64_t)tape.offsets[i];
    }
    p.T = T;
    if (count) p.input_lo = tape.offsets[0], p.input_hi = tape.offsets[count];
    make_tiles(p);
    EncodeRequest r{model, arena, (hipStream_t)stream, completion, scalar, embeddings, stats, trace, tape.data,
                    tape.offsets, count, outputs, states, token_vectors};
    run_encode(r, p, true);
}

}  // namespace

extern "C" void ube_image_encode_pixels(ube_image_encode_pixels_t *a) {
    if (!a) return;
    guarded(a->outcome, a->embeddings, a->states, a->token_vectors, a->arena, [&] {
        media_encode(a->model, a->arena, a->stream, a->completion, a->pixels, nullptr, a->heights, a->widths,
                     a->outputs_scalar, a->embeddings, a->stats, a->trace_residual, 2, a->outputs, a->states,
                     a->token_vectors);
    });
}

extern "C" void ube_video_encode_frames(ube_video_encode_frames_t *a) {
    if (!a) return;
    guarded(a->outcome, a->embeddings, a->states, a->token_vectors, a->arena, [&] {
        if (a->frames.count && !a->frame_counts) throw Failure{ube_status_invalid_argument_k, "NULL frame counts"};
        media_encode(a->model, a->arena, a->stream, a->completion, a->frames, a->frame_counts, a->heights, a->widths,
                     a->outputs_scalar, a->embeddings, a->stats, a->trace_residual, 3, a->outputs, a->states,
                     a->token_vectors);
    });
}

extern "C" void ube_maxsim(ube_maxsim_t *a) {
    if (!a) return;
    try {
        auto const &q = a->queries, &d = a->documents;
        if (!a->scores) throw Failure{ube_status_invalid_argument_k, "NULL scores"};
        if ((q.count && (!q.offsets || (q.rows && !q.data))) || (d.count && (!d.offsets || (d.rows && !d.data))))
            throw Failure{ube_status_invalid_argument_k, "NULL rows tape"};
        if (q.columns != d.columns) throw Failure{ube_status_invalid_argument_k, "queries and documents differ in width"};
        if (q.scalar != ube_scalar_bf16_k || d.scalar != ube_scalar_bf16_k)
            throw Failure{ube_status_unsupported_k, "MaxSim takes bf16 rows"};
        if (q.columns != 128 && q.columns != 256) throw Failure{ube_status_unsupported_k, "MaxSim width must be 128 or 256"};
        if (q.stride % 16 || d.stride % 16 || q.stride < q.columns * 2 || d.stride < d.columns * 2 ||
            ((uintptr_t)q.data % 16) || ((uintptr_t)d.data % 16))
            throw Failure{ube_status_invalid_argument_k, "rows must be 16-byte aligned and hold `columns` values"};
        if (q.count > 0x7fffffff || d.count > 0x7fffffff || q.count * d.count > ((size_t)1 << 40))
            throw Failure{ube_status_invalid_argument_k, "too many pairs"};
        const size_t ld = a->scores_stride ? a->scores_stride : d.count;
        if (ld < d.count) throw Failure{ube_status_invalid_argument_k, "scores_stride below the document count"};
        int ndev = 0;
        if (hipGetDeviceCount(&ndev) != hipSuccess || a->device < 0 || a->device >= ndev)
            throw Failure{ube_status_device_k, "no such GPU"};
        UBE_HIP(hipSetDevice(a->device));
        hipStream_t st = (hipStream_t)a->stream;
        const size_t span = a->query_span ? a->query_span : 64;
        UBE_HIP(launch_maxsim((const uint16_t *)q.data, q.offsets, q.rows, q.stride / 2, (int)q.count,
                              (const uint16_t *)d.data, d.offsets, d.rows, d.stride / 2, (int)d.count, (int)q.columns,
                              a->query_prefix, span, a->scores, ld, st));
        if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        set_outcome(a->outcome, f.status, f.message);
    }
}

// ============================================================== contrastive loss

namespace {

struct ResolvedEdges {
    std::vector<ContrastiveEdge> edges;     // sorted by (anchor, item)
    std::vector<uint32_t> row_edges;        // [R + 1]
    std::vector<uint32_t> col_offsets;      // [n + 1]
    std::vector<uint32_t> col_edges;        // [E]
    std::vector<uint32_t> touched;          // items with edges, ascending
};

// Reads one edge run; ids must be strictly ascending and name items.
void edge_run(ube_edges_view_t const &ev, size_t p, size_t n, size_t &lo, size_t &hi) {
    lo = hi = 0;
    if (!ev.offsets) return;
    lo = ev.offsets[p];
    hi = ev.offsets[p + 1];
    if (hi < lo) throw Failure{ube_status_invalid_argument_k, "edge offsets decrease"};
    if (hi > lo && !ev.ids) throw Failure{ube_status_invalid_argument_k, "NULL edge ids"};
    for (size_t e = lo; e < hi; ++e) {
        if (ev.ids[e] >= n) throw Failure{ube_status_invalid_argument_k, "edge names an item past the step"};
        if (e > lo && ev.ids[e] <= ev.ids[e - 1])
            throw Failure{ube_status_invalid_argument_k, "edge ids must ascend strictly within a run"};
    }
}

// Resolves the three edge sets per anchor in the pages' precedence (ignore, attract, repel), drops the
// item paired with itself, and drops ignore edges when no dense pass runs (they change nothing then).
ResolvedEdges resolve_edges(ube_relations_view_t const &rel, size_t r0, size_t R, size_t n, bool dense) {
    ResolvedEdges out;
    out.row_edges.assign(R + 1, 0);
    ube_edges_view_t const *sets[3] = {&rel.ignore, &rel.attract, &rel.repel};  // highest precedence first
    const int labels[3] = {0, 1, -1};
    for (size_t p = 0; p < R; ++p) {
        size_t lo[3], hi[3], at[3];
        for (int k = 0; k < 3; ++k) {
            edge_run(*sets[k], p, n, lo[k], hi[k]);
            at[k] = lo[k];
        }
        for (;;) {
            uint32_t j = UINT32_MAX;
            for (int k = 0; k < 3; ++k)
                if (at[k] < hi[k]) j = std::min(j, sets[k]->ids[at[k]]);
            if (j == UINT32_MAX) break;
            int label = 2;
            float w = 1.f;
            for (int k = 0; k < 3; ++k) {
                if (at[k] < hi[k] && sets[k]->ids[at[k]] == j) {
                    if (label == 2) {
                        label = labels[k];
                        if (labels[k] != 0 && sets[k]->weights) w = sets[k]->weights[at[k]];
                    }
                    ++at[k];
                }
            }
            if ((size_t)j == r0 + p) continue;
            if (label == 0 && !dense) continue;
            out.edges.push_back(ContrastiveEdge{(int)p, (int)j, label, w});
        }
        out.row_edges[p + 1] = (uint32_t)out.edges.size();
    }
    const size_t E = out.edges.size();
    if (!E) return out;
    out.col_offsets.assign(n + 1, 0);
    for (auto const &e : out.edges) ++out.col_offsets[e.j + 1];
    for (size_t j = 0; j < n; ++j) out.col_offsets[j + 1] += out.col_offsets[j];
    out.col_edges.resize(E);
    std::vector<uint32_t> fill(out.col_offsets.begin(), out.col_offsets.end() - 1);
    for (size_t e = 0; e < E; ++e) out.col_edges[fill[out.edges[e].j]++] = (uint32_t)e;
    std::vector<char> mark(n, 0);
    for (auto const &e : out.edges) mark[r0 + e.p] = mark[e.j] = 1;
    for (size_t i = 0; i < n; ++i)
        if (mark[i]) out.touched.push_back((uint32_t)i);
    return out;
}

}  // namespace

extern "C" void ube_contrastive(ube_contrastive_t *a) {
    if (!a) return;
    try {
        if (!a->arena) throw Failure{ube_status_invalid_argument_k, "NULL arena"};
        ArenaLease lease(a->arena);
        if (!lease.held) throw Failure{ube_status_contended_k, "arena busy"};
        ube_arena_t ar = a->arena;
        auto const &ev = a->embeddings;
        const size_t n = ev.count, D = ev.columns, R = a->anchor_count, r0 = a->anchor_begin;
        if (!a->scalars) throw Failure{ube_status_invalid_argument_k, "NULL scalars"};
        if (n && !ev.data) throw Failure{ube_status_invalid_argument_k, "NULL embeddings"};
        if (ev.scalar != ube_scalar_bf16_k) throw Failure{ube_status_unsupported_k, "contrastive loss takes bf16 rows"};
        if (D == 0 || D % 64 || D > 4096)
            throw Failure{ube_status_unsupported_k, "embedding width must be a multiple of 64 up to 4096"};
        if (ev.stride % 16 || ev.stride < D * 2 || ((uintptr_t)ev.data % 16))
            throw Failure{ube_status_invalid_argument_k, "rows must be 16-byte aligned and hold `columns` values"};
        if (n > ((size_t)1 << 30)) throw Failure{ube_status_invalid_argument_k, "too many items"};
        if (r0 > n || R > n - r0) throw Failure{ube_status_invalid_argument_k, "anchors outside the items"};
        if (a->negatives != ube_negatives_ambient_k && a->negatives != ube_negatives_named_k)
            throw Failure{ube_status_invalid_argument_k, "unknown negatives rule"};
        if (a->pair_loss != ube_pair_loss_form_derived_k && a->pair_loss != ube_pair_loss_form_sigmoid_k)
            throw Failure{ube_status_unsupported_k, "only the sigmoid pair loss runs here"};
        // widths
        std::vector<int> widths;
        if (!a->matryoshka_dimensions) {
            if (a->matryoshka_dimensions_count) throw Failure{ube_status_invalid_argument_k, "NULL widths"};
            widths.push_back((int)D);
        } else {
            if (a->matryoshka_dimensions_count == 0 || a->matryoshka_dimensions_count > (size_t)kMaxWidths)
                throw Failure{ube_status_invalid_argument_k, "between 1 and 8 widths"};
            for (size_t w = 0; w < a->matryoshka_dimensions_count; ++w) {
                const size_t m = a->matryoshka_dimensions[w];
                if (m == 0 || m % 8 || m > D || (w && m <= (size_t)widths.back()))
                    throw Failure{ube_status_invalid_argument_k,
                                  "widths must ascend strictly, be multiples of 8 and fit the rows"};
                widths.push_back((int)m);
            }
            for (int m : widths)
                if (m % 64) throw Failure{ube_status_unsupported_k, "widths must be multiples of 64 here"};
        }
        const int K = (int)widths.size();
        if (a->gradient && (a->gradient_stride % 16 || a->gradient_stride < D * 4 || ((uintptr_t)a->gradient % 16)))
            throw Failure{ube_status_invalid_argument_k, "gradient rows must be 16-byte aligned and hold `columns` floats"};
        if (n && !pointer_on_device(ev.data, ar->device))
            throw Failure{ube_status_device_k, "embeddings are not device memory of the arena's GPU"};
        if (n && ar->dev) {
            char const *lo = (char const *)ev.data, *hi = lo + (n - 1) * ev.stride + D * 2;
            if (hi > ar->dev && lo < ar->dev + ar->cap) throw Failure{ube_status_invalid_argument_k, "inputs lie inside the arena"};
        }
        UBE_HIP(hipSetDevice(ar->device));
        hipStream_t st = (hipStream_t)a->stream;
        const bool grad = a->gradient != nullptr;
        const bool dense = a->negatives == ube_negatives_ambient_k && a->ambient_repulsion_weight != 0.f;

        ContrastiveArgs ca{};
        ca.emb = (const uint16_t *)ev.data;
        ca.ld = ev.stride / 2;
        ca.n = (int)n;
        ca.R = (int)R;
        ca.r0 = (int)r0;
        ca.D = (int)D;
        ca.K = K;
        for (int w = 0; w < kMaxWidths; ++w) ca.widths[w] = w < K ? widths[w] : widths[K - 1];
        ca.t = a->inverse_temperature;
        ca.b = a->bias;
        ca.wa = a->ambient_repulsion_weight;
        ca.c = R ? 1.0f / (float)((double)K * (double)R) : 0.f;
        ca.dense = dense;
        ca.scalars = a->scalars;
        ca.want_loss = a->want_loss != 0;
        ca.grad = a->gradient;
        ca.gld = a->gradient_stride / 4;
        if (R == 0) {
            UBE_HIP(launch_contrastive_empty(ca, st));
            if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
            set_outcome(a->outcome, ube_status_success_k, nullptr);
            return;
        }
        ResolvedEdges re = resolve_edges(a->relations, r0, R, n, dense);
        const size_t E = re.edges.size(), T = re.touched.size();
        const size_t R_pad = align_up(R, 256), n_pad = align_up(n, 256);
        ca.R_pad = (int)R_pad;
        ca.n_pad = (int)n_pad;
        ca.E = (int)E;
        ca.T = (int)T;
        // split of the items for the rows contraction: about 512 workgroups
        const size_t per_split = (R_pad / 256) * (size_t)(widths[K - 1] / 64);
        size_t splits = std::max<size_t>(1, std::min<size_t>(n_pad / 64, (512 + per_split - 1) / per_split));
        const size_t chunk = align_up((n_pad + splits - 1) / splits, 64);
        splits = (n_pad + chunk - 1) / chunk;
        ca.splits = (int)splits;
        ca.chunk = (int)chunk;

        // workspace layout (256-byte aligned pieces)
        size_t off = 0;
        auto take = [&](size_t bytes) {
            size_t at = off;
            off += align_up(bytes, 256);
            return at;
        };
        const size_t JT = n_pad / 128, PT = R_pad / 128;
        const size_t o_inv = take((size_t)K * n * 4);
        const size_t o_h = take(grad && dense ? (size_t)K * R_pad * n_pad * 2 : 0);
        const size_t o_rowpart = take(dense ? JT * K * R_pad * 4 : 0);
        const size_t o_colpart = take(grad && dense ? PT * K * n_pad * 4 : 0);
        const size_t o_wg = take(dense ? PT * JT * K * 2 * 4 : 0);
        const size_t o_rho = take((size_t)K * R_pad * 4);
        const size_t o_kappa = take(grad ? (size_t)K * n_pad * 4 : 0);
        const size_t o_rsum = take((size_t)K * R_pad * 4);
        const size_t o_rpart = take(grad && dense ? splits * R_pad * D * 4 : 0);
        const size_t o_rfinal = take(grad && dense ? R_pad * D * 4 : 0);
        const size_t o_eout = take(E * 4 * K * 4);
        const size_t meta_begin = off;
        const size_t o_edges = take(E * sizeof(ContrastiveEdge));
        const size_t o_rowe = take(E ? (R + 1) * 4 : 0);
        const size_t o_colo = take(E ? (n + 1) * 4 : 0);
        const size_t o_cole = take(E * 4);
        const size_t o_touch = take(T * 4);
        const size_t total = off;
        arena_reserve(ar, total, st, false);
        char *db = ar->dev;
        ca.inv = (float *)(db + o_inv);
        ca.H = (uint16_t *)(db + o_h);
        ca.rowpart = (float *)(db + o_rowpart);
        ca.colpart = (float *)(db + o_colpart);
        ca.wgpart = (float *)(db + o_wg);
        ca.rho = (float *)(db + o_rho);
        ca.kappa_blk = (float *)(db + o_kappa);
        ca.rsum = (float *)(db + o_rsum);
        ca.rows_partial = (float *)(db + o_rpart);
        ca.rows_final = (float *)(db + o_rfinal);
        ca.edge_out = (float *)(db + o_eout);
        ca.edges = (const ContrastiveEdge *)(db + o_edges);
        ca.row_edges = (const uint32_t *)(db + o_rowe);
        ca.col_offsets = (const uint32_t *)(db + o_colo);
        ca.col_edges = (const uint32_t *)(db + o_cole);
        ca.touched = (const uint32_t *)(db + o_touch);

        // stage the resolved edges through the arena's pinned buffer
        const size_t meta_bytes = total - meta_begin;
        if (E) {
            if (ar->staged_pending) {
                UBE_HIP(hipEventSynchronize(ar->staged));
                ar->staged_pending = false;
            }
            if (meta_bytes > ar->pinned_cap) {
                if (ar->pinned) UBE_HIP(hipHostFree(ar->pinned));
                ar->pinned = nullptr;
                ar->pinned_cap = 0;
                const size_t want = align_up(meta_bytes, (size_t)1 << 16);
                UBE_HIP(hipHostMalloc((void **)&ar->pinned, want, 0));
                ar->pinned_cap = want;
            }
            if (!ar->staged) UBE_HIP(hipEventCreateWithFlags(&ar->staged, hipEventDisableTiming));
            char *hp = ar->pinned;
            std::memcpy(hp + (o_edges - meta_begin), re.edges.data(), E * sizeof(ContrastiveEdge));
            std::memcpy(hp + (o_rowe - meta_begin), re.row_edges.data(), (R + 1) * 4);
            std::memcpy(hp + (o_colo - meta_begin), re.col_offsets.data(), (n + 1) * 4);
            std::memcpy(hp + (o_cole - meta_begin), re.col_edges.data(), E * 4);
            std::memcpy(hp + (o_touch - meta_begin), re.touched.data(), T * 4);
            UBE_HIP(hipMemcpyAsync(db + meta_begin, hp, meta_bytes, hipMemcpyHostToDevice, st));
            UBE_HIP(hipEventRecord(ar->staged, st));
            ar->staged_pending = true;
        }

        UBE_HIP(launch_prefix_inv_norms(ca, st));
        UBE_HIP(launch_contrastive_edges(ca, st));
        timed(ube_kernel_contrastive_cells_k, st, [&] { return launch_contrastive_cells(ca, grad, st); });
        UBE_HIP(launch_contrastive_reduce(ca, grad, st));
        if (grad) {
            timed(ube_kernel_contrastive_rows_k, st, [&] { return launch_contrastive_grad_rows(ca, st); });
            timed(ube_kernel_contrastive_cols_k, st, [&] { return launch_contrastive_grad_cols(ca, st); });
            UBE_HIP(launch_contrastive_sparse(ca, st));
        }
        if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        set_outcome(a->outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        set_outcome(a->outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

extern "C" char const *ube_status_name(ube_status_t s) {
    switch (s) {
        case ube_status_success_k: return "success";
        case ube_status_invalid_argument_k: return "invalid_argument";
        case ube_status_shape_mismatch_k: return "shape_mismatch";
        case ube_status_out_of_memory_k: return "out_of_memory";
        case ube_status_device_k: return "device";
        case ube_status_contended_k: return "contended";
        case ube_status_unsupported_k: return "unsupported";
        case ube_status_internal_k: return "internal";
    }
    return "unknown";
}

// ===================================================================== trainer

namespace {
// Workspace of one training forward and backward over T tokens: the activations the forward keeps (k*),
// host-built tables (cu, tiles, positions, byte -> token lists), then the backward's scratch.
struct TrainLayout {
    size_t kx, kx1, kqk, kvt, ko, klse, kgu, kxf, ks, kcu, ktiles, kpos, tok_off, tok;
    size_t h1, h2, gu, dx, dxb, da, dgu, act, dh, dx1, dx1b, dout, dqkv, gpart, gsum, xty, dz, pd, z,
        du, spa, zpart, dupart, dxf, delta, total;
    size_t Tpad, rows_per_block;
};
}  // namespace

struct ube_trainer_handle_t {
    ube_model_t model = nullptr;
    int device = 0;
    float beta1 = 0.9f, decay = -0.8f, eps1 = 1e-30f, clip = 1.0f;
    size_t step = 0;
    char *mem = nullptr;  // masters, derived packings, gradients, optimizer state
    size_t bytes = 0;
    struct Tensor {
        char const *name;
        size_t layer, rows, cols;  // cols == 0: a vector of `rows`
        uint16_t *w16 = nullptr;   // bf16 master (matrices, the pool query)
        float *w32 = nullptr;      // fp32 master (norm gains)
        float *grad = nullptr, *r = nullptr, *c = nullptr, *v = nullptr, *m = nullptr;
    };
    std::vector<Tensor> tensors;
    struct Block {  // indices into tensors, and packings derived from the masters
        size_t qkv, o, gate, up, down, g1, g2;
        uint16_t *guT, *gu_cols, *qkvT;  // qkvT: recomputation only
    };
    std::vector<Block> blocks;
    size_t t_embed = 0, t_gf = 0, t_query = 0, t_wk = 0, t_wv = 0;
    // device tables of the multi-tensor update and of the repacking, with their grid sizes
    ube::AdaTensor *ada_table = nullptr;
    int ada_stats = 0, ada_cols = 0, ada_upd = 0;
    ube::PackJob *pack_table = nullptr;
    int pack_jobs = 0, pack_wgs = 0;
    // activation recomputation: the forward keeps only each block's fp32 input and the backward replays
    // the block from it (else the forward keeps every activation the backward reads)
    bool recompute = false;
    // the last training forward, whose activations the workspace holds until a step changes the weights
    bool fw_valid = false;
    size_t fw_T = 0, fw_count = 0, fw_ntiles = 0;
    TrainLayout fw_L{};
    // per-call workspace (grows)
    char *ws = nullptr;
    size_t ws_cap = 0;
};

namespace {

// The forward keeps each block's gate/up pre-activations unless activations are recomputed (a trainer's
// ffn is a multiple of 128, so the gate/up product always runs on the 256-column tiles that store them).
bool keeps_gate_up(ube_geometry_t const &g, bool recompute) { return !recompute && (2 * g.ffn) % 256 == 0; }

TrainLayout train_carve(ube_geometry_t const &g, size_t T, size_t count, size_t ntiles, bool recompute) {
    TrainLayout L{};
    const size_t D = g.hidden, F = g.ffn, H = g.heads, N = g.depth;
    L.Tpad = align_up(T, 256) + kRowPad;
    const size_t Tp = L.Tpad, T1 = std::max<size_t>(T, 1);
    size_t total = 0;
    auto take = [&](size_t bytes) {
        size_t o = total;
        total = align_up(total + bytes, 256);
        return o;
    };
    // kept by the forward (recomputation: one block's set, refilled by each block's replay)
    const size_t NB = recompute ? 1 : N;
    L.kx = take((N + 1) * T1 * D * 4);
    L.kx1 = take(NB * T1 * D * 4);
    L.kqk = take(NB * Tp * 2 * D * 2);
    L.kvt = take(NB * D * Tp * 2);
    L.ko = take(NB * Tp * D * 2);
    L.klse = take(NB * H * Tp * 4);
    const bool kgu = keeps_gate_up(g, recompute);
    L.kgu = take(kgu ? N * Tp * 2 * F * 2 : 0);
    L.kxf = take(Tp * D * 2);
    L.ks = take(Tp * H * 4);
    L.kcu = take((count + 1) * 4);
    L.ktiles = take(std::max<size_t>(ntiles, 1) * 8);
    L.kpos = take(Tp * 4 * 2);
    L.tok_off = take((g.vocab + 1) * 4);
    L.tok = take(T1 * 4);
    // backward scratch
    L.h1 = take(Tp * D * 2);
    L.h2 = take(Tp * D * 2);
    L.gu = take(kgu ? 0 : Tp * 2 * F * 2);  // rebuilt per block when not kept
    L.dx = take(Tp * D * 4);
    L.dxb = take(Tp * D * 2);
    L.da = take(Tp * F * 2);
    L.dgu = take(Tp * 2 * F * 2);
    L.act = take(Tp * F * 2);
    L.dh = take(Tp * D * 4);
    L.dx1 = take(Tp * D * 4);
    L.dx1b = take(Tp * D * 2);
    L.dout = take(Tp * D * 2);
    L.dqkv = take(Tp * 3 * D * 2);
    L.delta = take(H * Tp * 4);
    L.rows_per_block = 64;
    const size_t gblocks = (size_t)rmsnorm_bwd_blocks((int)T1, (int)L.rows_per_block);
    L.gpart = take(gblocks * D * 4);
    L.gsum = take((gblocks + 31) / 32 * D * 4);
    // weight-gradient partials: ranges of tokens for each product's shape
    size_t xty_floats = 0;
    for (auto mn : {std::array<size_t, 2>{D, 3 * D}, {D, D}, {D, 2 * F}, {F, D}}) {
        int sp = 0, ch = 0;
        xty_split((int)T1, (int)mn[0], (int)mn[1], &sp, &ch);
        xty_floats = std::max(xty_floats, (size_t)sp * mn[0] * mn[1]);
    }
    L.xty = take(xty_floats * 4);
    L.dz = take(std::max<size_t>(count, 1) * H * D * 4);
    L.pd = take(Tp * H * 2 * 4);
    L.z = take(std::max<size_t>(count, 1) * H * D * 4);
    L.du = take(std::max<size_t>(count, 1) * H * D * 4);
    L.spa = take(std::max<size_t>(count, 1) * (size_t)pool_bwd_token_ranges((int)count) * H * 4);
    const size_t pchunks = (size_t)pool_bwd_chunks((int)count);
    L.zpart = take(std::max<size_t>(count, 1) * pchunks * H * D * 4);
    L.dupart = take(std::max<size_t>(count, 1) * pchunks * H * D * 4);
    L.dxf = take(Tp * D * 4);
    L.total = total;
    return L;
}

// GEMM y = x W with W given as [N x K] K-contiguous (the kernels' packed layout)
void gemm(int epi, const uint16_t *w, const uint16_t *x, int M, int N, int K, uint16_t *out_bf16, int ld_out,
          float *out_f32, int ld_f32, hipStream_t st) {
    GemmArgs ga{};
    ga.w = w, ga.x = x, ga.M = M, ga.N = N, ga.K = K;
    ga.out_bf16 = out_bf16, ga.ld_out = ld_out, ga.out_f32 = out_f32, ga.ld_f32 = ld_f32, ga.scale = 1.0f;
    UBE_HIP(launch_gemm(epi, ga, st));
}

// Derived packings after the masters change (one launch over the job table): the trainer's unfolded
// gate/up copies, the model's forward weights (gains folded, pool keys refolded) and its plain copies.
void repack(ube_trainer_t tr, hipStream_t st) {
    UBE_HIP(launch_pack(tr->pack_table, tr->pack_jobs, tr->pack_wgs, st));
}

}  // namespace

extern "C" void ube_trainer_init(ube_trainer_init_t *a) {
    if (!a) return;
    if (a->trainer) *a->trainer = nullptr;
    ube_trainer_t tr = nullptr;
    try {
        if (!a->trainer || !a->model || !a->weights) throw Failure{ube_status_invalid_argument_k, "NULL trainer, model or weights"};
        ube_model_t m = a->model;
        const ube_geometry_t &g = m->g;
        if (!m->text) throw Failure{ube_status_unsupported_k, "training runs text models"};
        if (m->e4m3) throw Failure{ube_status_unsupported_k, "training runs bf16 models (E4M3 is inference-only)"};
        if (g.rope_axes != 1) throw Failure{ube_status_unsupported_k, "training runs 1-axis rotary"};
        if (g.hidden > 1024 || g.hidden % 128 || g.heads > 16 || g.ffn % 128)
            throw Failure{ube_status_unsupported_k, "training runs hidden <= 1024 and ffn, multiples of 128"};
        ube_weights_t const &w = *a->weights;
        if (!w.embed || !w.w_qkv || !w.w_o || !w.w_gate || !w.w_up || !w.w_down || !w.attn_norm || !w.mlp_norm ||
            !w.final_norm || !w.pool_query || !w.pool_wk || !w.pool_wv)
            throw Failure{ube_status_invalid_argument_k, "missing weights"};
        UBE_HIP(hipSetDevice(m->device));
        const size_t D = g.hidden, F = g.ffn, N = g.depth, V = g.vocab;
        tr = new ube_trainer_handle_t();
        tr->model = m;
        tr->device = m->device;
        if (a->beta1 > 0.f) tr->beta1 = a->beta1;
        if (a->decay_rate < 0.f) tr->decay = a->decay_rate;
        if (a->epsilon1 > 0.f) tr->eps1 = a->epsilon1;
        if (a->clip_threshold > 0.f) tr->clip = a->clip_threshold;
        tr->recompute = a->activation_recomputation != 0;
        // tensors in a fixed order: embed, blocks, final gain, pool query, W_k, W_v
        auto add = [&](char const *name, size_t layer, size_t rows, size_t cols) {
            tr->tensors.push_back(ube_trainer_handle_t::Tensor{name, layer, rows, cols});
            return tr->tensors.size() - 1;
        };
        tr->t_embed = add("embed", 0, V, D);
        tr->blocks.resize(N);
        for (size_t l = 0; l < N; ++l) {
            auto &b = tr->blocks[l];
            b.g1 = add("attn_norm", l, D, 0);
            b.qkv = add("w_qkv", l, D, 3 * D);
            b.o = add("w_o", l, D, D);
            b.g2 = add("mlp_norm", l, D, 0);
            b.gate = add("w_gate", l, D, F);
            b.up = add("w_up", l, D, F);
            b.down = add("w_down", l, F, D);
        }
        tr->t_gf = add("final_norm", 0, D, 0);
        tr->t_query = add("pool_query", 0, D, 0);
        tr->t_wk = add("pool_wk", 0, D, D);
        tr->t_wv = add("pool_wv", 0, D, D);
        // device memory
        size_t total = 0;
        auto take = [&](size_t bytes) {
            size_t o = total;
            total = align_up(total + bytes, 256);
            return o;
        };
        std::vector<std::array<size_t, 6>> offs(tr->tensors.size());
        for (size_t i = 0; i < tr->tensors.size(); ++i) {
            auto const &t = tr->tensors[i];
            const size_t n = t.rows * (t.cols ? t.cols : 1);
            const bool fp32_master = t.cols == 0 && std::strcmp(t.name, "pool_query") != 0;
            offs[i][0] = take(n * (fp32_master ? 4 : 2));
            offs[i][1] = take(n * 4);                    // gradient
            offs[i][2] = take(t.cols ? t.rows * 4 : 0);  // r
            offs[i][3] = take(t.cols ? t.cols * 4 : 0);  // c
            offs[i][4] = take(t.cols ? 0 : n * 4);       // v
            offs[i][5] = take(n * 4);                    // m
        }
        std::vector<std::array<size_t, 3>> aoffs(tr->tensors.size());  // col_parts, rms_parts, mean_r
        for (size_t i = 0; i < tr->tensors.size(); ++i) {
            auto const &t = tr->tensors[i];
            const size_t n = t.rows * (t.cols ? t.cols : 1);
            aoffs[i] = {take(t.cols ? (t.rows + kAdaSlice - 1) / kAdaSlice * t.cols * 4 : 0),
                        take((n + kAdaChunk - 1) / kAdaChunk * 4), take(4)};
        }
        std::vector<std::array<size_t, 3>> boffs(N);
        for (size_t l = 0; l < N; ++l)
            boffs[l] = {take(2 * F * D * 2), take(2 * F * D * 2), take(tr->recompute ? 3 * D * D * 2 : 0)};
        const size_t n_jobs = 9 * N + 4;
        const size_t o_ada = take(tr->tensors.size() * sizeof(AdaTensor));
        const size_t o_pack = take(n_jobs * sizeof(PackJob));
        UBE_HIP(hipMalloc((void **)&tr->mem, total));
        tr->bytes = total;
        UBE_HIP(hipMemset(tr->mem, 0, total));
        char *db = tr->mem;
        for (size_t i = 0; i < tr->tensors.size(); ++i) {
            auto &t = tr->tensors[i];
            const bool fp32_master = t.cols == 0 && std::strcmp(t.name, "pool_query") != 0;
            if (fp32_master) t.w32 = (float *)(db + offs[i][0]);
            else t.w16 = (uint16_t *)(db + offs[i][0]);
            t.grad = (float *)(db + offs[i][1]);
            t.r = t.cols ? (float *)(db + offs[i][2]) : nullptr;
            t.c = t.cols ? (float *)(db + offs[i][3]) : nullptr;
            t.v = t.cols ? nullptr : (float *)(db + offs[i][4]);
            t.m = (float *)(db + offs[i][5]);
        }
        for (size_t l = 0; l < N; ++l) {
            auto &b = tr->blocks[l];
            b.guT = (uint16_t *)(db + boffs[l][0]);
            b.gu_cols = (uint16_t *)(db + boffs[l][1]);
            b.qkvT = tr->recompute ? (uint16_t *)(db + boffs[l][2]) : nullptr;
        }
        // the multi-tensor update's table
        std::vector<AdaTensor> ada(tr->tensors.size());
        for (size_t i = 0; i < tr->tensors.size(); ++i) {
            auto const &t = tr->tensors[i];
            AdaTensor &e = ada[i];
            e.g = t.grad, e.w16 = t.w16, e.w32 = t.w32, e.r = t.r, e.c = t.c, e.v = t.v, e.m = t.m;
            e.col_parts = (float *)(db + aoffs[i][0]), e.rms_parts = (float *)(db + aoffs[i][1]);
            e.mean_r = (float *)(db + aoffs[i][2]);
            e.rows = (int)t.rows, e.cols = (int)t.cols;
        }
        if (adafactor_grids(ada.data(), (int)ada.size(), &tr->ada_stats, &tr->ada_cols, &tr->ada_upd) != 0)
            throw Failure{ube_status_unsupported_k, "a tensor of 2^31 elements or more"};
        tr->ada_table = (AdaTensor *)(db + o_ada);
        UBE_HIP(hipMemcpy(tr->ada_table, ada.data(), ada.size() * sizeof(AdaTensor), hipMemcpyHostToDevice));
        // the repacking's jobs
        {
            auto &T = tr->tensors;
            const int Di = (int)D, Fi = (int)F, Hi = (int)g.heads;
            std::vector<PackJob> jobs;
            auto job = [&](const void *src, const void *src2, const float *gain, void *dst, int K, int Nn, int kind) {
                jobs.push_back(PackJob{src, src2, gain, dst, K, Nn, kind, 0});
            };
            for (size_t l = 0; l < N; ++l) {
                auto const &b = tr->blocks[l];
                auto &ml = m->layers[l];
                job(T[b.gate].w16, T[b.up].w16, nullptr, b.guT, Di, Fi, kPackTransposePair);
                job(T[b.gate].w16, T[b.up].w16, nullptr, b.gu_cols, Di, Fi, kPackColumnPair);
                job(T[b.qkv].w16, nullptr, T[b.g1].w32, ml.wqkv, Di, 3 * Di, kPackTranspose);
                job(T[b.o].w16, nullptr, nullptr, ml.wo, Di, Di, kPackTranspose);
                job(T[b.gate].w16, T[b.up].w16, T[b.g2].w32, ml.wgu, Di, Fi, kPackTransposePair);
                job(T[b.down].w16, nullptr, nullptr, ml.wd, Fi, Di, kPackTranspose);
                job(T[b.g1].w32, nullptr, nullptr, ml.g1, 1, Di, kPackCopy);
                job(T[b.g2].w32, nullptr, nullptr, ml.g2, 1, Di, kPackCopy);
                if (b.qkvT) job(T[b.qkv].w16, nullptr, nullptr, b.qkvT, Di, 3 * Di, kPackTranspose);
            }
            job(T[tr->t_embed].w16, nullptr, nullptr, m->embed, 1, (int)(V * D / 2), kPackCopy);
            job(T[tr->t_gf].w32, nullptr, nullptr, m->gf, 1, Di, kPackCopy);
            job(T[tr->t_wv].w16, nullptr, nullptr, m->wv, 1, Di * Di / 2, kPackCopy);
            job(T[tr->t_wk].w16, T[tr->t_query].w16, nullptr, m->u, Di, Hi, kPackPoolKeys);
            if (jobs.size() > n_jobs) throw Failure{ube_status_invalid_argument_k, "packing table overflow"};
            tr->pack_wgs = pack_workgroups(jobs.data(), (int)jobs.size());
            tr->pack_jobs = (int)jobs.size();
            tr->pack_table = (PackJob *)(db + o_pack);
            UBE_HIP(hipMemcpy(tr->pack_table, jobs.data(), jobs.size() * sizeof(PackJob), hipMemcpyHostToDevice));
        }
        // masters from the caller's canonical weights
        auto up16 = [&](size_t i, uint16_t const *src) {
            auto const &t = tr->tensors[i];
            UBE_HIP(hipMemcpy(t.w16, src, t.rows * (t.cols ? t.cols : 1) * 2, hipMemcpyHostToDevice));
        };
        auto up32 = [&](size_t i, float const *src) {
            UBE_HIP(hipMemcpy(tr->tensors[i].w32, src, tr->tensors[i].rows * 4, hipMemcpyHostToDevice));
        };
        up16(tr->t_embed, w.embed);
        for (size_t l = 0; l < N; ++l) {
            auto const &b = tr->blocks[l];
            up32(b.g1, w.attn_norm[l]);
            up16(b.qkv, w.w_qkv[l]);
            up16(b.o, w.w_o[l]);
            up32(b.g2, w.mlp_norm[l]);
            up16(b.gate, w.w_gate[l]);
            up16(b.up, w.w_up[l]);
            up16(b.down, w.w_down[l]);
        }
        up32(tr->t_gf, w.final_norm);
        up16(tr->t_query, w.pool_query);
        up16(tr->t_wk, w.pool_wk);
        up16(tr->t_wv, w.pool_wv);
        repack(tr, nullptr);
        UBE_HIP(hipDeviceSynchronize());
        *a->trainer = tr;
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        if (tr) {
            if (tr->mem) (void)hipFree(tr->mem);
            delete tr;
        }
        set_outcome(a->outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        if (tr) {
            if (tr->mem) (void)hipFree(tr->mem);
            delete tr;
        }
        set_outcome(a->outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

extern "C" void ube_trainer_free(ube_trainer_t tr) {
    if (!tr) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(tr->device);
    (void)hipDeviceSynchronize();
    if (tr->mem) (void)hipFree(tr->mem);
    if (tr->ws) (void)hipFree(tr->ws);
    (void)hipSetDevice(prev);
    delete tr;
}

extern "C" size_t ube_trainer_tensors(ube_trainer_t tr, ube_trainer_tensor_t *out, size_t capacity) {
    if (!tr) return 0;
    for (size_t i = 0; i < tr->tensors.size() && i < capacity && out; ++i) {
        auto const &t = tr->tensors[i];
        out[i] = ube_trainer_tensor_t{t.name, t.layer, t.rows, t.cols, t.w16 ? (void *)t.w16 : (void *)t.w32,
                                      t.w16 ? ube_scalar_bf16_k : ube_scalar_f32_k, t.grad};
    }
    return tr->tensors.size();
}

namespace {

// The training forward over a byte tape: the model's forward (pooled fp32 rows into the arena) with the
// activations of the backward kept in the trainer's workspace, plus the tables the backward reads
// (item bounds, tiles, positions, and the tokens of every byte value in token order).
void train_forward(ube_trainer_t tr, ube_arena_t arena, hipStream_t st, ube_tape_view_t const &texts,
                   ube_encode_stats_t *stats, ube_rows_view_t *rows) {
    ube_model_t m = tr->model;
    const ube_geometry_t &g = m->g;
    if (arena->device != tr->device) throw Failure{ube_status_device_k, "arena and trainer on different GPUs"};
    const size_t V = g.vocab;
    tr->fw_valid = false;
    Plan p = text_plan(m, texts);
    const size_t T = p.T, count = texts.count;
    UBE_HIP(hipSetDevice(tr->device));
    // byte of every kept token, grouped by value in token order (the embedding gradient's fixed order)
    std::vector<uint8_t> bytes(p.input_hi - p.input_lo);
    if (!bytes.empty()) {
        const bool dev = pointer_on_device(texts.data, tr->device);
        const char *src = (const char *)texts.data + p.input_lo;
        if (dev) UBE_HIP(hipMemcpy(bytes.data(), src, bytes.size(), hipMemcpyDeviceToHost));
        else std::memcpy(bytes.data(), src, bytes.size());
    }
    std::vector<uint32_t> tok_off(V + 1, 0), tok(std::max<size_t>(T, 1));
    for (size_t i = 0; i < count; ++i)
        for (int t = p.cu[i]; t < p.cu[i + 1]; ++t) ++tok_off[bytes[p.src[i] - p.input_lo + (t - p.cu[i])] + 1];
    for (size_t v = 0; v < V; ++v) tok_off[v + 1] += tok_off[v];
    {
        std::vector<uint32_t> fill(tok_off.begin(), tok_off.end() - 1);
        for (size_t i = 0; i < count; ++i)
            for (int t = p.cu[i]; t < p.cu[i + 1]; ++t)
                tok[fill[bytes[p.src[i] - p.input_lo + (t - p.cu[i])]]++] = (uint32_t)t;
    }
    TrainLayout L = train_carve(g, T, count, p.tiles.size(), tr->recompute);
    if (L.total > tr->ws_cap) {
        UBE_HIP(hipStreamSynchronize(st));
        if (tr->ws) UBE_HIP(hipFree(tr->ws));
        tr->ws = nullptr;
        tr->ws_cap = 0;
        const size_t want = align_up(L.total, (size_t)1 << 20);
        UBE_HIP(hipMalloc((void **)&tr->ws, want));
        tr->ws_cap = want;
        UBE_HIP(hipMemsetAsync(tr->ws, 0, want, st));
    }
    char *wb = tr->ws;
    UBE_HIP(hipMemcpyAsync(wb + L.tok_off, tok_off.data(), (V + 1) * 4, hipMemcpyHostToDevice, st));
    UBE_HIP(hipMemcpyAsync(wb + L.tok, tok.data(), tok.size() * 4, hipMemcpyHostToDevice, st));
    Keep k{};
    k.x = (float *)(wb + L.kx), k.xf = (uint16_t *)(wb + L.kxf), k.s = (float *)(wb + L.ks);
    if (!tr->recompute) {
        k.x1 = (float *)(wb + L.kx1);
        k.qk = (uint16_t *)(wb + L.kqk), k.vt = (uint16_t *)(wb + L.kvt), k.o = (uint16_t *)(wb + L.ko);
        k.lse = (float *)(wb + L.klse);
        if (keeps_gate_up(g, false)) k.gu = (uint16_t *)(wb + L.kgu);
    }
    k.Tpad = L.Tpad, k.ldvt = L.Tpad, k.ldl = L.Tpad;
    Layout EL{};
    EncodeRequest r{m, arena, st, 1, ube_scalar_f32_k, rows, stats, nullptr, texts.data, texts.offsets, count, 0,
                    nullptr, nullptr, &EL, &k};
    run_encode(r, p, false);
    char *ab = arena->dev;
    if (T) {
        UBE_HIP(hipMemcpyAsync(wb + L.kcu, ab + EL.cu, (count + 1) * 4, hipMemcpyDeviceToDevice, st));
        // the attention's launch order: the trainer's tile list serves its attention kernels only
        UBE_HIP(hipMemcpyAsync(wb + L.ktiles, ab + EL.atiles, p.tiles.size() * 8, hipMemcpyDeviceToDevice, st));
        UBE_HIP(hipMemcpyAsync(wb + L.kpos, ab + EL.pos, L.Tpad * 4 * 2, hipMemcpyDeviceToDevice, st));
    }
    tr->fw_T = T, tr->fw_count = count, tr->fw_ntiles = p.tiles.size(), tr->fw_L = L;
    tr->fw_valid = true;
}

// The backward over the last training forward's activations: d loss / d every parameter from d loss /
// d pooled rows. Per block (last to first) the few inputs that were not kept are rebuilt from the kept
// rows (the two RMSNorm outputs, v's rows, the gate/up pre-activations), then the block's backward runs.
void train_backward(ube_trainer_t tr, hipStream_t st, float const *d_embeddings) {
    ube_model_t m = tr->model;
    const ube_geometry_t &g = m->g;
    const size_t D = g.hidden, F = g.ffn, H = g.heads, N = g.depth, V = g.vocab;
    const float eps = g.rms_epsilon;
    const TrainLayout &L = tr->fw_L;
    const size_t T = tr->fw_T, count = tr->fw_count;
    UBE_HIP(hipSetDevice(tr->device));
    if (T == 0) {
        for (auto const &t : tr->tensors) UBE_HIP(hipMemsetAsync(t.grad, 0, t.rows * (t.cols ? t.cols : 1) * 4, st));
        return;
    }
    char *wb = tr->ws;
    auto F32 = [&](size_t o) { return (float *)(wb + o); };
    auto B16 = [&](size_t o) { return (uint16_t *)(wb + o); };
    const int *cu = (const int *)(wb + L.kcu);
    const int2 *tiles = (const int2 *)(wb + L.ktiles);
    const int ntiles = (int)tr->fw_ntiles;
    const int16_t *pos = (const int16_t *)(wb + L.kpos);
    auto &TT = tr->tensors;
    const int Ti = (int)T, Di = (int)D, Fi = (int)F, Hi = (int)H;
    const size_t Tp = L.Tpad, TD = T * D;
    const int ldvt = (int)Tp, ldl = (int)Tp;
    const int blocks = rmsnorm_bwd_blocks(Ti, (int)L.rows_per_block);
    auto xty = [&](const uint16_t *x, int M, const uint16_t *y, int Nn, float *out, float *out2, bool di) {
        timed(ube_kernel_weight_grad_k, st, [&] {
            return launch_xty(x, M, y, Nn, Ti, M, Nn, F32(L.xty), out, out2, di,
                              st);
        });
    };
    // ---- pool and final norm
    PoolBwdArgs pa{};
    pa.xf = B16(L.kxf), pa.s = F32(L.ks), pa.cu = cu, pa.count = (int)count, pa.D = Di, pa.H = Hi, pa.u = m->u;
    pa.wv = TT[tr->t_wv].w16, pa.wk = TT[tr->t_wk].w16, pa.query = TT[tr->t_query].w16;
    pa.dpooled = d_embeddings;
    pa.dxf = F32(L.dxf), pa.z = F32(L.z), pa.du = F32(L.du);
    pa.dwv = TT[tr->t_wv].grad, pa.dwk = TT[tr->t_wk].grad, pa.dquery = TT[tr->t_query].grad;
    UBE_HIP(launch_pool_bwd(pa, F32(L.dz), F32(L.pd), F32(L.spa), F32(L.zpart), F32(L.dupart), st));
    UBE_HIP(launch_rmsnorm_bwd(F32(L.kx) + N * TD, TT[tr->t_gf].w32, F32(L.dxf), nullptr, F32(L.dx), B16(L.dxb),
                               F32(L.gpart), (int)L.rows_per_block, Ti, Di, eps, st));
    UBE_HIP(launch_sum_rows(F32(L.gpart), blocks, Di, TT[tr->t_gf].grad, F32(L.gsum), st));
    // ---- blocks, last to first
    for (size_t li = N; li-- > 0;) {
        auto const &b = tr->blocks[li];
        const size_t kb = tr->recompute ? 0 : li;  // which kept set holds this block's activations
        const float *x_in = F32(L.kx) + li * TD;
        float *x1 = F32(L.kx1) + kb * TD;
        uint16_t *qk = B16(L.kqk) + kb * Tp * 2 * D, *vt = B16(L.kvt) + kb * D * Tp, *o = B16(L.ko) + kb * Tp * D;
        float *lse = F32(L.klse) + kb * H * Tp;
        uint16_t *h1 = B16(L.h1), *h2 = B16(L.h2), *gu = B16(L.gu);
        float *delta = F32(L.delta);
        UBE_HIP(launch_rmsnorm(x_in, TT[b.g1].w32, h1, Ti, Di, eps, st));
        if (tr->recompute) {
            // replay the block's attention half from its fp32 input
            UBE_HIP(hipMemset2DAsync(vt + T, (size_t)ldvt * 2, 0, 64 * 2, D, st));
            GemmArgs qa{};
            qa.w = b.qkvT, qa.x = h1, qa.M = Ti, qa.N = 3 * Di, qa.K = Di;
            qa.out_bf16 = qk, qa.ld_out = 2 * Di, qa.vt = vt, qa.ld_vt = ldvt, qa.pos = pos, qa.rope = m->rope;
            qa.D = Di, qa.sec0 = m->sec0, qa.sec1 = m->sec1;
            UBE_HIP(launch_gemm(kEpiQkv, qa, st));
            UBE_HIP(launch_attention(qk, qk + D, 2 * Di, vt, ldvt, o, Di, cu, tiles, ntiles, Hi, st, lse, ldl));
            GemmArgs oa{};
            oa.w = m->layers[li].wo, oa.x = o, oa.M = Ti, oa.N = Di, oa.K = Di;
            oa.out_f32 = x1, oa.ld_f32 = Di, oa.res_in = x_in, oa.scale = 1.0f;
            UBE_HIP(launch_gemm(kEpiResid, oa, st));
        }
        // the block's inputs that were not kept (v is read feature-major, as kept)
        UBE_HIP(launch_rmsnorm(x1, TT[b.g2].w32, h2, Ti, Di, eps, st));
        if (!keeps_gate_up(g, tr->recompute))
            gemm(kEpiStore, b.guT, h2, Ti, 2 * Fi, Di, gu, 2 * Fi, nullptr, 0, st);
        else
            gu = B16(L.kgu) + li * Tp * 2 * F;  // kept by the forward's gate/up product
        // MLP half
        float *dx = F32(L.dx), *dh = F32(L.dh), *dx1 = F32(L.dx1);
        uint16_t *dxb = B16(L.dxb), *da = B16(L.da), *dgu = B16(L.dgu), *act = B16(L.act), *dx1b = B16(L.dx1b);
        gemm(kEpiStore, TT[b.down].w16, dxb, Ti, Fi, Di, da, Fi, nullptr, 0, st);
        UBE_HIP(launch_swiglu_bwd(gu, da, dgu, act, Ti, Fi, st));
        xty(act, Fi, dxb, Di, TT[b.down].grad, nullptr, false);
        gemm(kEpiPatch, b.gu_cols, dgu, Ti, Di, 2 * Fi, nullptr, 0, dh, Di, st);
        xty(h2, Di, dgu, 2 * Fi, TT[b.gate].grad, TT[b.up].grad, true);
        UBE_HIP(launch_rmsnorm_bwd(x1, TT[b.g2].w32, dh, dx, dx1, dx1b, F32(L.gpart), (int)L.rows_per_block, Ti, Di,
                                   eps, st));
        UBE_HIP(launch_sum_rows(F32(L.gpart), blocks, Di, TT[b.g2].grad, F32(L.gsum), st));
        // attention half
        uint16_t *dout = B16(L.dout), *dqkv = B16(L.dqkv);
        gemm(kEpiStore, TT[b.o].w16, dx1b, Ti, Di, Di, dout, Di, nullptr, 0, st);
        xty(o, Di, dx1b, Di, TT[b.o].grad, nullptr, false);
        AttnBwdArgs ab2{};
        ab2.q = qk, ab2.k = qk + D, ab2.ldqk = 2 * Di, ab2.vt = vt, ab2.ldvt = ldvt, ab2.dout = dout, ab2.lddo = Di;
        ab2.lse = lse, ab2.delta = delta, ab2.ldl = ldl, ab2.o = o, ab2.ldo = Di;
        ab2.dq = dqkv, ab2.dk = dqkv + D, ab2.dv = dqkv + 2 * D, ab2.ldd = 3 * Di;  // straight into d[q|k|v]
        ab2.cu = cu, ab2.tiles = tiles, ab2.ntiles = ntiles, ab2.heads = Hi, ab2.pos = pos, ab2.rope = m->rope;
        timed(ube_kernel_attention_bwd_k, st, [&] { return launch_attention_bwd(ab2, st); });
        gemm(kEpiPatch, TT[b.qkv].w16, dqkv, Ti, Di, 3 * Di, nullptr, 0, dh, Di, st);
        xty(h1, Di, dqkv, 3 * Di, TT[b.qkv].grad, nullptr, false);
        UBE_HIP(launch_rmsnorm_bwd(x_in, TT[b.g1].w32, dh, dx1, dx, dxb, F32(L.gpart), (int)L.rows_per_block, Ti, Di,
                                   eps, st));
        UBE_HIP(launch_sum_rows(F32(L.gpart), blocks, Di, TT[b.g1].grad, F32(L.gsum), st));
    }
    UBE_HIP(launch_embed_bwd(F32(L.dx), (const uint32_t *)(wb + L.tok_off), (const uint32_t *)(wb + L.tok), (int)V, Di,
                             TT[tr->t_embed].grad, st));
}

}  // namespace

extern "C" void ube_trainer_forward(ube_trainer_forward_t *a) {
    if (!a) return;
    if (a->embeddings) *a->embeddings = ube_rows_view_t{nullptr, 0, 0, 0, ube_scalar_unknown_k};
    try {
        if (!a->trainer || !a->arena) throw Failure{ube_status_invalid_argument_k, "NULL trainer or arena"};
        if (!a->embeddings) throw Failure{ube_status_invalid_argument_k, "NULL embeddings output"};
        ArenaLease lease(a->arena);
        if (!lease.held) throw Failure{ube_status_contended_k, "the arena is serving another call"};
        hipStream_t st = (hipStream_t)a->stream;
        train_forward(a->trainer, a->arena, st, a->texts, a->stats, a->embeddings);
        if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        if (a->trainer) a->trainer->fw_valid = false;
        if (a->embeddings) *a->embeddings = ube_rows_view_t{nullptr, 0, 0, 0, ube_scalar_unknown_k};
        set_outcome(a->outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        if (a->trainer) a->trainer->fw_valid = false;
        set_outcome(a->outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

extern "C" void ube_trainer_backward(ube_trainer_backward_t *a) {
    if (!a) return;
    try {
        if (!a->trainer) throw Failure{ube_status_invalid_argument_k, "NULL trainer"};
        ube_trainer_t tr = a->trainer;
        const size_t D = tr->model->g.hidden;
        hipStream_t st = (hipStream_t)a->stream;
        if (a->after_forward) {
            if (!tr->fw_valid)
                throw Failure{ube_status_invalid_argument_k, "no training forward since the last step"};
        } else {
            if (!a->arena) throw Failure{ube_status_invalid_argument_k, "NULL arena"};
            ArenaLease lease(a->arena);
            if (!lease.held) throw Failure{ube_status_contended_k, "the arena is serving another call"};
            ube_rows_view_t rows{};
            train_forward(tr, a->arena, st, a->texts, a->stats, &rows);
        }
        if (tr->fw_count && !a->d_embeddings) throw Failure{ube_status_invalid_argument_k, "NULL embedding gradient"};
        if (tr->fw_count && a->d_embeddings_stride && a->d_embeddings_stride != D * 4)
            throw Failure{ube_status_unsupported_k, "embedding gradient rows must be packed"};
        train_backward(tr, st, a->d_embeddings);
        if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        set_outcome(a->outcome, f.status, f.message);
    } catch (std::bad_alloc const &) {
        set_outcome(a->outcome, ube_status_out_of_memory_k, "host out of memory");
    }
}

extern "C" void ube_trainer_step(ube_trainer_step_t *a) {
    if (!a) return;
    try {
        if (!a->trainer) throw Failure{ube_status_invalid_argument_k, "NULL trainer"};
        ube_trainer_t tr = a->trainer;
        UBE_HIP(hipSetDevice(tr->device));
        hipStream_t st = (hipStream_t)a->stream;
        tr->step += 1;
        tr->fw_valid = false;  // the kept activations belong to the weights before this update
        const double t = (double)tr->step;
        const float beta2 = (float)(1.0 - std::pow(t, (double)tr->decay));
        const float bc = (float)(1.0 - std::pow((double)tr->beta1, t));
        AdaStep as{a->learning_rate, tr->beta1, beta2, tr->eps1, tr->clip, bc};
        UBE_HIP(launch_adafactor(tr->ada_table, (int)tr->tensors.size(), tr->ada_stats, tr->ada_cols, tr->ada_upd, as,
                                 st));
        repack(tr, st);
        if (a->completion == 0) UBE_HIP(hipStreamSynchronize(st));
        set_outcome(a->outcome, ube_status_success_k, nullptr);
    } catch (Failure const &f) {
        set_outcome(a->outcome, f.status, f.message);
    }
}

// ===================================================================== steps

namespace {
ube_status_t step_status(hipError_t e) {
    if (e == hipSuccess) return ube_status_success_k;
    if (e == hipErrorInvalidValue) return ube_status_invalid_argument_k;
    return ube_status_device_k;
}
}  // namespace

extern "C" ube_status_t ube_step_gemm(void const *w, void const *x, void *y, size_t M, size_t N, size_t K,
                                      void *stream) {
    if (!w || !x || !y || N % 128 || K % 64 || !N || !K || M > 0x7fffffff) return ube_status_invalid_argument_k;
    GemmArgs a{};
    a.w = (const uint16_t *)w, a.x = (const uint16_t *)x, a.M = (int)M, a.N = (int)N, a.K = (int)K;
    a.out_bf16 = (uint16_t *)y, a.ld_out = (int)N;
    return step_status(launch_gemm(kEpiStore, a, (hipStream_t)stream));
}

extern "C" ube_status_t ube_step_qkv_rotary(void const *w, void const *x, size_t M, size_t D, size_t K,
                                           int16_t const *pos_host, size_t rope_axes, float rope_base,
                                           size_t positions, void *qk, void *vt, size_t ldvt, void *stream) {
    if (!w || !x || !qk || !vt || (M && !pos_host) || !D || D % 128 || !K || K % 64 || rope_axes < 1 ||
        rope_axes > 3 || !positions || positions > 32767 || M > 0x7fffff00 || D > 8192 ||
        ldvt < align_up(M, 256) || ldvt > 0x7fffffff)
        return ube_status_invalid_argument_k;
    for (size_t t = 0; t < M; ++t)
        for (size_t a = 0; a < 3; ++a)
            if (pos_host[t * 4 + a] < 0 || (size_t)pos_host[t * 4 + a] >= positions) return ube_status_invalid_argument_k;
    std::vector<float2> table(positions * 32);
    for (size_t p = 0; p < positions; ++p)
        for (int j = 0; j < 32; ++j) {
            const double phi = (double)p * std::pow((double)rope_base, -2.0 * (double)j / 64.0);
            table[p * 32 + j] = float2{(float)std::cos(phi), (float)std::sin(phi)};
        }
    hipStream_t st = (hipStream_t)stream;
    void *drope = nullptr, *dpos = nullptr;
    hipError_t e = hipMalloc(&drope, table.size() * sizeof(float2));
    if (e == hipSuccess) e = hipMalloc(&dpos, std::max<size_t>(M, 1) * 8);
    if (e == hipSuccess) e = hipMemcpyAsync(drope, table.data(), table.size() * sizeof(float2), hipMemcpyHostToDevice, st);
    if (e == hipSuccess && M) e = hipMemcpyAsync(dpos, pos_host, M * 8, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) {
        GemmArgs a{};
        a.w = (const uint16_t *)w, a.x = (const uint16_t *)x, a.M = (int)M, a.N = (int)(3 * D), a.K = (int)K;
        a.out_bf16 = (uint16_t *)qk, a.ld_out = (int)(2 * D), a.vt = (uint16_t *)vt, a.ld_vt = (int)ldvt;
        a.pos = (const int16_t *)dpos, a.rope = (const float2 *)drope, a.D = (int)D;
        const int pairs = 32, axes = (int)rope_axes, base = pairs / axes, rem = pairs % axes;
        a.sec0 = base + (0 < rem ? 1 : 0);
        a.sec1 = axes >= 2 ? base + (1 < rem ? 1 : 0) : 0;
        e = launch_gemm(kEpiQkv, a, st);
    }
    // the 256-wide kernel writes the columns past M as zeros itself; the narrow one leaves them
    const size_t Mp = align_up(M, 256);
    if (e == hipSuccess && Mp > M) e = hipMemset2DAsync((char *)vt + M * 2, ldvt * 2, 0, (Mp - M) * 2, D, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (drope) (void)hipFree(drope);
    if (dpos) (void)hipFree(dpos);
    return step_status(e);
}

extern "C" ube_status_t ube_step_quantize_e4m3(void const *in, void *codes, float *scales, size_t T, size_t W,
                                               void *stream) {
    if (!in || !codes || !scales || W % 8 || !W || T > 0x7fffffff || W > 0x7fffffff) return ube_status_invalid_argument_k;
    return step_status(launch_quantize_rows((const uint16_t *)in, (uint8_t *)codes, scales, (int)T, (int)W,
                                            (hipStream_t)stream));
}

extern "C" ube_status_t ube_step_gemm_e4m3(void const *w, float w_scale, void const *x, float const *x_scale, void *y,
                                           size_t M, size_t N, size_t K, void *stream) {
    if (!w || !x || !x_scale || !y || N % 256 || K % 128 || !N || !K || M > 0x7fffffff)
        return ube_status_invalid_argument_k;
    GemmArgs a{};
    a.w = (const uint16_t *)w, a.x = (const uint16_t *)x, a.M = (int)M, a.N = (int)N, a.K = (int)K;
    a.out_bf16 = (uint16_t *)y, a.ld_out = (int)N, a.x_scale = x_scale, a.w_scale = w_scale;
    return step_status(launch_gemm_e4m3(kEpiStore, a, (hipStream_t)stream));
}

extern "C" ube_status_t ube_step_rmsnorm(float const *x, float const *gain, void *h, size_t T, size_t D, float eps,
                                         void *stream) {
    if (!x || !gain || !h || !row_width_supported(D) || T > 0x7fffffff) return ube_status_invalid_argument_k;
    return step_status(launch_rmsnorm(x, gain, (uint16_t *)h, (int)T, (int)D, eps, (hipStream_t)stream));
}

extern "C" ube_status_t ube_step_attention(void const *q, void const *k, size_t ldqk, void const *vt, size_t ldvt,
                                           void *o, size_t ldo, uint32_t const *cu_host, size_t count, size_t heads,
                                           void *stream) {
    if (!q || !k || !vt || !o || !cu_host || !heads) return ube_status_invalid_argument_k;
    std::vector<int> cu(count + 1);
    Plan p;
    p.count = count;
    for (size_t i = 0; i <= count; ++i) {
        if (i && cu_host[i] < cu_host[i - 1]) return ube_status_invalid_argument_k;
        cu[i] = (int)cu_host[i];
    }
    p.cu = cu;
    make_tiles(p);
    if (ldvt < (size_t)cu[count] + kRowPad) return ube_status_invalid_argument_k;
    void *dcu = nullptr, *dtiles = nullptr;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMalloc(&dcu, (count + 1) * 4);
    if (e == hipSuccess) e = hipMalloc(&dtiles, std::max<size_t>(p.tiles.size(), 1) * 8);
    if (e == hipSuccess) e = hipMemcpyAsync(dcu, cu.data(), (count + 1) * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess && !p.tiles.empty())
        e = hipMemcpyAsync(dtiles, p.tiles.data(), p.tiles.size() * 8, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = launch_attention((const uint16_t *)q, (const uint16_t *)k, (int)ldqk, (const uint16_t *)vt, (int)ldvt,
                             (uint16_t *)o, (int)ldo, (const int *)dcu, (const int2 *)dtiles, (int)p.tiles.size(),
                             (int)heads, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (dcu) (void)hipFree(dcu);
    if (dtiles) (void)hipFree(dtiles);
    return step_status(e);
}

extern "C" ube_status_t ube_kernel_timer_start(ube_kernel_t kernel, size_t max_launches) {
    if ((int)kernel < 0 || kernel >= ube_kernel_count_k || !max_launches) return ube_status_invalid_argument_k;
    std::lock_guard<std::mutex> lock(g_timer.mu);
    for (hipEvent_t e : g_timer.events) (void)hipEventDestroy(e);
    g_timer.events.clear();
    g_timer.used = 0;
    g_timer.kernel = -1;
    for (size_t i = 0; i < 2 * max_launches; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            for (hipEvent_t d : g_timer.events) (void)hipEventDestroy(d);
            g_timer.events.clear();
            return ube_status_device_k;
        }
        g_timer.events.push_back(e);
    }
    g_timer.kernel = (int)kernel;
    return ube_status_success_k;
}

extern "C" ube_status_t ube_kernel_timer_stop(double *total_ms, size_t *launches) {
    std::lock_guard<std::mutex> lock(g_timer.mu);
    double total = 0.0;
    ube_status_t status = ube_status_success_k;
    for (size_t i = 0; i + 1 < g_timer.used; i += 2) {
        float ms = 0.f;
        if (hipEventSynchronize(g_timer.events[i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_timer.events[i], g_timer.events[i + 1]) != hipSuccess) {
            status = ube_status_device_k;
            break;
        }
        total += ms;
    }
    if (total_ms) *total_ms = total;
    if (launches) *launches = g_timer.used / 2;
    for (hipEvent_t e : g_timer.events) (void)hipEventDestroy(e);
    g_timer.events.clear();
    g_timer.used = 0;
    g_timer.kernel = -1;
    return status;
}

extern "C" char const *ube_kernel_name(ube_kernel_t k) {
    static char const *names[] = {"gather",       "patchify",  "rmsnorm",    "gemm_patch", "gemm_qkv", "attention",
                                  "gemm_out",     "gemm_gate_up", "gemm_down", "final_norm", "pool",     "quantize",
                                  "contrastive_cells", "contrastive_rows", "contrastive_cols", "attention_bwd",
                                  "weight_grad"};
    return ((int)k >= 0 && k < ube_kernel_count_k) ? names[k] : "unknown";
}
