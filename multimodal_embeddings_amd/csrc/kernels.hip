// kernels.hip -- gfx950 kernels of the uniform byte encoder's forward pass.
//
// Steps (UForm documentation, "UForm" page, "Architecture & Goals" and
// "Precision by Design"): byte gather, RMSNorm, QKV projection with multi-axis
// rotary positions, bidirectional varlen attention, output projection and
// residual, RMSNorm, SwiGLU MLP and residual, final RMSNorm, attention pooling
// ("UForm" page, FAQ "Why attention pooling instead of mean pooling?").
// Storage is bf16, accumulation and normalisation fp32, the residual stream fp32.
//
// MFMA: v_mfma_f32_32x32x16_bf16. Lane l of a wave supplies row (l % 32) of the
// A operand and column (l % 32) of the B operand, each as 8 consecutive k values
// of half (l / 32); both operands use the same (half, slot) -> k assignment, so
// any consistent k permutation gives the same product. The 32x32 fp32 result
// sits in lane l, register r = 4i + j at row 8i + 4(l / 32) + j, column l % 32.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace ube {


// =========================================================== row kernels
//
// One wave per token row. Lane l holds features c*64*V + l*V + [0, V) for
// chunks c < C (D = 64*V*C): coalesced 64*V-float spans per chunk.

template <int V>
struct RowIO;

template <>
struct RowIO<2> {
    __device__ static void load_f32(const float *p, float *v) {
        f32x2 a = *(const f32x2 *)p;
        v[0] = a.x, v[1] = a.y;
    }
    __device__ static void store_f32(float *p, const float *v) { *(f32x2 *)p = f32x2{v[0], v[1]}; }
    __device__ static void load_bf16(const uint16_t *p, float *v) {
        uint32_t a = *(const uint32_t *)p;
        v[0] = bf16_to_f32(a & 0xffff), v[1] = bf16_to_f32(a >> 16);
    }
    __device__ static void store_bf16(uint16_t *p, const float *v) { *(uint32_t *)p = pack2(v[0], v[1]); }
};

template <>
struct RowIO<4> {
    __device__ static void load_f32(const float *p, float *v) {
        f32x4 a = *(const f32x4 *)p;
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
    }
    __device__ static void store_f32(float *p, const float *v) { *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]}; }
    __device__ static void load_bf16(const uint16_t *p, float *v) {
        u32x2 a = *(const u32x2 *)p;
        v[0] = bf16_to_f32(a.x & 0xffff), v[1] = bf16_to_f32(a.x >> 16);
        v[2] = bf16_to_f32(a.y & 0xffff), v[3] = bf16_to_f32(a.y >> 16);
    }
    __device__ static void store_bf16(uint16_t *p, const float *v) {
        *(u32x2 *)p = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
    }
};

template <>
struct RowIO<8> {
    __device__ static void load_f32(const float *p, float *v) {
        RowIO<4>::load_f32(p, v);
        RowIO<4>::load_f32(p + 4, v + 4);
    }
    __device__ static void store_f32(float *p, const float *v) {
        RowIO<4>::store_f32(p, v);
        RowIO<4>::store_f32(p + 4, v + 4);
    }
    __device__ static void load_bf16(const uint16_t *p, float *v) {
        u32x4 a = *(const u32x4 *)p;
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) v[2 * i] = bf16_to_f32(w[i] & 0xffff), v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    __device__ static void store_bf16(uint16_t *p, const float *v) {
        *(u32x4 *)p = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
    }
};

// x row (fp32, in registers) -> h = bf16(x * g / sqrt(mean(x^2) + eps)).
template <int V, int C>
__device__ __forceinline__ void norm_store(float (&v)[C][V], const float *gain, uint16_t *hrow, int D, float eps,
                                           int lane) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < V; ++i) ss += v[c][i] * v[c][i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int f = c * 64 * V + lane * V;
        float g[V], o[V];
        if constexpr (V == 2) {
            f32x2 gg = *(const f32x2 *)(gain + f);
            g[0] = gg.x, g[1] = gg.y;
        } else {
#pragma unroll
            for (int i = 0; i < V; i += 4) {
                f32x4 gg = *(const f32x4 *)(gain + f + i);
                g[i] = gg.x, g[i + 1] = gg.y, g[i + 2] = gg.z, g[i + 3] = gg.w;
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = v[c][i] * inv * g[i];
        RowIO<V>::store_bf16(hrow + f, o);
    }
}

template <int V, int C>
__global__ __launch_bounds__(256) void k_gather_text(const uint8_t *__restrict__ data, const int64_t *__restrict__ src,
                                                     const int *__restrict__ cu, const int2 *__restrict__ tiles,
                                                     const uint16_t *__restrict__ embed, float *__restrict__ x,
                                                     uint16_t *__restrict__ xb, float *__restrict__ ss,
                                                     int16_t *__restrict__ pos, int D) {
    const int2 tile = tiles[blockIdx.x];
    const int item = tile.x, start = cu[item], end = min(tile.y + kTileTokens, cu[item + 1]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t = tile.y + wave; t < end; t += 4) {
        const int local = t - start;
        const uint32_t byte = data[src[item] + local];
        float v[V];
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int f = c * 64 * V + lane * V;
            RowIO<V>::load_bf16(embed + (size_t)byte * D + f, v);
            RowIO<V>::store_f32(x + (size_t)t * D + f, v);
            RowIO<V>::store_bf16(xb + (size_t)t * D + f, v);  // exact: embedding rows are bf16
#pragma unroll
            for (int i = 0; i < V; ++i) sq += v[i] * v[i];
        }
        sq = wave_sum(sq);
        if (lane < kSsParts) ss[(size_t)t * kSsParts + lane] = lane == 0 ? sq : 0.f;
        if (lane == 0) *(u32x2 *)(pos + (size_t)t * 4) = u32x2{(uint32_t)(local & 0xffff), 0u};
    }
}

template <int V, int C>
__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, const float *__restrict__ gain,
                                                 uint16_t *__restrict__ h, int T, int D, float eps) {
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += waves) {
        float v[C][V];
#pragma unroll
        for (int c = 0; c < C; ++c) RowIO<V>::load_f32(x + (size_t)t * D + c * 64 * V + lane * V, v[c]);
        norm_store<V, C>(v, gain, h + (size_t)t * D, D, eps, lane);
    }
}

// Final RMSNorm and pool scores, R rows per wave at a time: the R rows' loads are
// in flight together and their reductions interleave, so a wave is not left
// waiting on one row's load and one row's chain of cross-lane steps at a time.
// Pool scores s[t][h] = xf_t . u_h for up to HP heads, the per-lane partial dots of
// all heads reduced across lanes together (lanes_reduce); each u value read from
// LDS serves all R rows.
template <int V, int C, int HP>
__global__ __launch_bounds__(256) void k_final_norm_scores(const float *__restrict__ x, const float *__restrict__ gain,
                                                           const float *__restrict__ u, uint16_t *__restrict__ xf,
                                                           float *__restrict__ s, float *__restrict__ states, int T,
                                                           int D, int H, float eps) {
    constexpr int R = 4;
    // u [H x D] in LDS with each lane's V consecutive values spread one per bank row: value i of lane l in
    // column group c sits at 64 V c + 64 i + l, so a wave reading value i of all its lanes touches 64
    // consecutive dwords (in u's own order, lanes V floats apart, eight lanes would share each bank)
    // (filled in LDS order, so consecutive threads write consecutive dwords and gather from u, a few KB in L2)
    extern __shared__ float su[];
    for (int d = threadIdx.x; d < H * D; d += 256) {
        const int hd = d / D, r = d % D, c = r / (64 * V), i = (r / 64) % V, l = r % 64;
        su[d] = u[hd * D + c * 64 * V + l * V + i];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    float g[C][V];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < V; ++i) g[c][i] = gain[c * 64 * V + lane * V + i];
    for (int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R; t0 < T; t0 += waves * R) {
        float v[R][C][V], ss[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ss[r] = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (t0 + r < T) {
                    RowIO<V>::load_f32(x + (size_t)(t0 + r) * D + c * 64 * V + lane * V, v[r][c]);
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i) v[r][c][i] = 0.f;
                }
#pragma unroll
                for (int i = 0; i < V; ++i) ss[r] += v[r][c][i] * v[r][c][i];
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
            for (int r = 0; r < R; ++r) ss[r] += __shfl_xor(ss[r], m, 64);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float inv = 1.0f / sqrtf(ss[r] / (float)D + eps);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int f = c * 64 * V + lane * V;
#pragma unroll
                for (int i = 0; i < V; ++i) v[r][c][i] = v[r][c][i] * inv * g[c][i];
                if (t0 + r < T) {
                    RowIO<V>::store_bf16(xf + (size_t)(t0 + r) * D + f, v[r][c]);
                    if (states) RowIO<V>::store_f32(states + (size_t)(t0 + r) * D + f, v[r][c]);
                }
            }
        }
        float dots[R][HP];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int hd = 0; hd < HP; ++hd) dots[r][hd] = 0.f;
#pragma unroll
        for (int hd = 0; hd < HP; ++hd) {
            if (hd < H) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        const float uv = su[hd * D + c * 64 * V + i * 64 + lane];
#pragma unroll
                        for (int r = 0; r < R; ++r) dots[r][hd] += v[r][c][i] * uv;
                    }
                }
            }
        }
        constexpr int LPH = 64 / HP;  // lanes per head after the reduction
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float tot = lanes_reduce<HP>(dots[r], lane);
            if (t0 + r < T && lane % LPH == 0 && lane / LPH < H) s[(size_t)(t0 + r) * H + lane / LPH] = tot;
        }
    }
}

// ------------------------------------------------------------- E4M3 rows
//
// Per-row activation quantisation for the E4M3 GEMMs: scale = amax / 448, code
// = OCP E4M3 of value * 448 / amax (v_cvt_pk_fp8_f32: nearest even; |values| stay
// within 448). An all-zero row gets scale 0 and zero codes.

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);       // bytes 2, 3
    return (uint32_t)w;
}

// RMSNorm straight to E4M3 codes and a per-row scale.
template <int V, int C>
__global__ __launch_bounds__(256) void k_rmsnorm_e4m3(const float *__restrict__ x, const float *__restrict__ gain,
                                                      uint8_t *__restrict__ h8, float *__restrict__ hs, int T, int D,
                                                      float eps) {
    static_assert(V % 4 == 0 || V == 2, "");
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += waves) {
        float v[C][V];
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            RowIO<V>::load_f32(x + (size_t)t * D + c * 64 * V + lane * V, v[c]);
#pragma unroll
            for (int i = 0; i < V; ++i) ss += v[c][i] * v[c][i];
        }
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)D + eps);
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < V; ++i) {
                v[c][i] = v[c][i] * inv * gain[c * 64 * V + lane * V + i];
                amax = fmaxf(amax, fabsf(v[c][i]));
            }
        amax = wave_max(amax);
        const float q = amax > 0.f ? 448.0f / amax : 0.f;
        if (lane == 0) hs[t] = amax / 448.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            uint8_t *dst = h8 + (size_t)t * D + c * 64 * V + lane * V;
            if constexpr (V == 2) {
                const uint32_t w = pack4_e4m3(v[c][0] * q, v[c][1] * q, 0.f, 0.f);
                *(uint16_t *)dst = (uint16_t)(w & 0xffff);
            } else {
#pragma unroll
                for (int i = 0; i < V; i += 4)
                    *(uint32_t *)(dst + i) = pack4_e4m3(v[c][i] * q, v[c][i + 1] * q, v[c][i + 2] * q, v[c][i + 3] * q);
            }
        }
    }
}

// bf16 rows [T x W] -> E4M3 codes + per-row scales; one wave per row, W % 8 == 0.
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t *__restrict__ in, uint8_t *__restrict__ out,
                                                       float *__restrict__ scale, int T, int W) {
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += waves) {
        const uint16_t *row = in + (size_t)t * W;
        float amax = 0.f;
        for (int e = lane * 8; e < W; e += 512) {
            float v[8];
            RowIO<8>::load_bf16(row + e, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        }
        amax = wave_max(amax);
        const float q = amax > 0.f ? 448.0f / amax : 0.f;
        if (lane == 0) scale[t] = amax / 448.0f;
        for (int e = lane * 8; e < W; e += 512) {
            float v[8];
            RowIO<8>::load_bf16(row + e, v);
            *(u32x2 *)(out + (size_t)t * W + e) =
                u32x2{pack4_e4m3(v[0] * q, v[1] * q, v[2] * q, v[3] * q), pack4_e4m3(v[4] * q, v[5] * q, v[6] * q, v[7] * q)};
        }
    }
}

// (V, C) with D = 64*V*C, C <= 8.
#define UBE_ROW_DISPATCH(D, ...)                         \
    do {                                                         \
        const int _n = (D) / 128;                                \
        if ((D) % 512 == 0 && (D) / 512 <= 8) {                  \
            switch ((D) / 512) {                                 \
                case 1: { constexpr int V = 8, C = 1; __VA_ARGS__; } break; \
                case 2: { constexpr int V = 8, C = 2; __VA_ARGS__; } break; \
                case 3: { constexpr int V = 8, C = 3; __VA_ARGS__; } break; \
                case 4: { constexpr int V = 8, C = 4; __VA_ARGS__; } break; \
                default: return hipErrorInvalidValue;            \
            }                                                    \
        } else if ((D) % 256 == 0) {                             \
            switch ((D) / 256) {                                 \
                case 1: { constexpr int V = 4, C = 1; __VA_ARGS__; } break; \
                case 3: { constexpr int V = 4, C = 3; __VA_ARGS__; } break; \
                case 5: { constexpr int V = 4, C = 5; __VA_ARGS__; } break; \
                case 7: { constexpr int V = 4, C = 7; __VA_ARGS__; } break; \
                default: return hipErrorInvalidValue;            \
            }                                                    \
        } else {                                                 \
            switch (_n) {                                        \
                case 1: { constexpr int V = 2, C = 1; __VA_ARGS__; } break; \
                case 3: { constexpr int V = 2, C = 3; __VA_ARGS__; } break; \
                case 5: { constexpr int V = 2, C = 5; __VA_ARGS__; } break; \
                case 7: { constexpr int V = 2, C = 7; __VA_ARGS__; } break; \
                default: return hipErrorInvalidValue;            \
            }                                                    \
        }                                                        \
    } while (0)

hipError_t launch_gather_text(const uint8_t *data, const int64_t *src, const int *cu, const int2 *tiles,
                              int ntiles, const uint16_t *embed, float *x, uint16_t *xb, float *ss, int16_t *pos,
                              int D, hipStream_t stream) {
    if (ntiles == 0) return hipSuccess;
    UBE_ROW_DISPATCH(D, (k_gather_text<V, C><<<ntiles, 256, 0, stream>>>(data, src, cu, tiles, embed, x, xb, ss, pos,
                                                                           D)));
    return hipGetLastError();
}

static int row_grid(int T) {
    int blocks = (T + 3) / 4;
    return blocks < 8192 ? blocks : 8192;
}

hipError_t launch_rmsnorm_e4m3(const float *x, const float *gain, uint8_t *h8, float *hs, int T, int D, float eps,
                               hipStream_t stream) {
    if (T == 0) return hipSuccess;
    UBE_ROW_DISPATCH(D, (k_rmsnorm_e4m3<V, C><<<row_grid(T), 256, 0, stream>>>(x, gain, h8, hs, T, D, eps)));
    return hipGetLastError();
}

// The same for rows of NV * 512 values: the row's loads are all issued before the maximum is taken, and the
// codes are formed from the registers (one read of the row).
template <int NV>
__global__ __launch_bounds__(256) void k_quantize_rows_fixed(const uint16_t *__restrict__ in, uint8_t *__restrict__ out,
                                                             float *__restrict__ scale, int T) {
    constexpr int W = NV * 512;
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += waves) {
        const uint16_t *row = in + (size_t)t * W;
        float v[NV][8];
#pragma unroll
        for (int c = 0; c < NV; ++c) RowIO<8>::load_bf16(row + c * 512 + lane * 8, v[c]);
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
        amax = wave_max(amax);
        const float q = amax > 0.f ? 448.0f / amax : 0.f;
        if (lane == 0) scale[t] = amax / 448.0f;
#pragma unroll
        for (int c = 0; c < NV; ++c)
            *(u32x2 *)(out + (size_t)t * W + c * 512 + lane * 8) =
                u32x2{pack4_e4m3(v[c][0] * q, v[c][1] * q, v[c][2] * q, v[c][3] * q),
                      pack4_e4m3(v[c][4] * q, v[c][5] * q, v[c][6] * q, v[c][7] * q)};
    }
}

hipError_t launch_quantize_rows(const uint16_t *in, uint8_t *out, float *scale, int T, int W, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    if (W % 8) return hipErrorInvalidValue;
    switch (W % 512 == 0 ? W / 512 : 0) {
        case 1: k_quantize_rows_fixed<1><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        case 2: k_quantize_rows_fixed<2><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        case 3: k_quantize_rows_fixed<3><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        case 4: k_quantize_rows_fixed<4><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        case 6: k_quantize_rows_fixed<6><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        case 8: k_quantize_rows_fixed<8><<<row_grid(T), 256, 0, stream>>>(in, out, scale, T); break;
        default: k_quantize_rows<<<row_grid(T), 256, 0, stream>>>(in, out, scale, T, W); break;
    }
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *x, const float *gain, uint16_t *h, int T, int D, float eps,
                          hipStream_t stream) {
    if (T == 0) return hipSuccess;
    UBE_ROW_DISPATCH(D, (k_rmsnorm<V, C><<<row_grid(T), 256, 0, stream>>>(x, gain, h, T, D, eps)));
    return hipGetLastError();
}

hipError_t launch_final_norm_scores(const float *x, const float *gain, const float *u, uint16_t *xf, float *s,
                                    float *states, int T, int D, int H, float eps, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const size_t lds = (size_t)H * D * sizeof(float);
    // four rows per wave: a quarter of the row kernels' grid, and no more workgroups than fit on the CUs
    // at once (each first copies u, up to 64 KB, into LDS; the waves then stride over the rows)
    const int resident = 256 * (int)std::max<size_t>(1, (160 * 1024) / lds);
    const int grid = std::min(row_grid((T + 3) / 4), resident);
    auto run = [&](auto kernel) -> hipError_t {
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        kernel<<<grid, 256, lds, stream>>>(x, gain, u, xf, s, states, T, D, H, eps);
        return hipSuccess;
    };
    UBE_ROW_DISPATCH(D, {
        const hipError_t e = H <= 8 ? run(k_final_norm_scores<V, C, 8>) : run(k_final_norm_scores<V, C, 16>);
        if (e != hipSuccess) return e;
    });
    return hipGetLastError();
}

// Token vectors: every fp32 row divided by its Euclidean norm (a zero row stays
// zero), written as f32 or bf16.
template <int V, int C>
__global__ __launch_bounds__(256) void k_unit_rows(const float *__restrict__ in, void *__restrict__ out, int out_bf16,
                                                   int T, int W) {
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += waves) {
        float v[C][V];
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            RowIO<V>::load_f32(in + (size_t)t * W + c * 64 * V + lane * V, v[c]);
#pragma unroll
            for (int i = 0; i < V; ++i) ss += v[c][i] * v[c][i];
        }
        ss = wave_sum(ss);
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int f = c * 64 * V + lane * V;
#pragma unroll
            for (int i = 0; i < V; ++i) v[c][i] *= inv;
            if (out_bf16)
                RowIO<V>::store_bf16((uint16_t *)out + (size_t)t * W + f, v[c]);
            else
                RowIO<V>::store_f32((float *)out + (size_t)t * W + f, v[c]);
        }
    }
}

hipError_t launch_unit_rows(const float *in, void *out, int out_bf16, int T, int W, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    UBE_ROW_DISPATCH(W, (k_unit_rows<V, C><<<row_grid(T), 256, 0, stream>>>(in, out, out_bf16, T, W)));
    return hipGetLastError();
}

// =========================================================== patchify
//
// Token (f, r, c) of an item: the 16x16x3 patch at grid (r, c) of frame f,
// element k = (py*16 + px)*3 + ch = pixel(16r + py, 16c + px, ch). One wave per
// token; lane l writes elements [12 l, 12 l + 12): py = l / 4, px = 4 (l % 4) + [0, 4).
__global__ __launch_bounds__(256) void k_patchify(const uint8_t *__restrict__ pixels,
                                                  const MediaItem *__restrict__ items, const int *__restrict__ cu,
                                                  const int2 *__restrict__ tiles, uint16_t *__restrict__ patches,
                                                  int16_t *__restrict__ pos, int axes) {
    const int2 tile = tiles[blockIdx.x];
    const MediaItem it = items[tile.x];
    const int start = cu[tile.x], end = min(tile.y + kTileTokens, cu[tile.x + 1]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_frame = it.grid_h * it.grid_w;
    const size_t frame_bytes = (size_t)per_frame * 256 * 3;
    for (int t = tile.y + wave; t < end; t += 4) {
        const int local = t - start;
        const int f = local / per_frame, rem = local % per_frame;
        const int r = rem / it.grid_w, c = rem % it.grid_w;
        const int py = lane >> 2, px = (lane & 3) * 4;
        const uint8_t *p = pixels + it.pixel_offset + (size_t)f * frame_bytes +
                           ((size_t)(16 * r + py) * it.width + 16 * c + px) * 3;
        uint32_t w[6];
        // bf16 of a byte value is exact; two per word
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const float a = (float)p[2 * i], b = (float)p[2 * i + 1];
            w[i] = pack2(a, b);
        }
        uint16_t *out = patches + (size_t)t * 768 + lane * 12;
        *(u32x2 *)(out + 0) = u32x2{w[0], w[1]};
        *(u32x2 *)(out + 4) = u32x2{w[2], w[3]};
        *(u32x2 *)(out + 8) = u32x2{w[4], w[5]};
        if (lane == 0) {
            const int p0 = axes == 3 ? f : r, p1 = axes == 3 ? r : c, p2 = axes == 3 ? c : 0;
            *(u32x2 *)(pos + (size_t)t * 4) =
                u32x2{(uint32_t)(p0 & 0xffff) | ((uint32_t)(p1 & 0xffff) << 16), (uint32_t)(p2 & 0xffff)};
        }
    }
}

hipError_t launch_patchify(const uint8_t *pixels, const MediaItem *items, const int *cu, const int2 *tiles,
                           int ntiles, uint16_t *patches, int16_t *pos, int axes, hipStream_t stream) {
    if (ntiles == 0) return hipSuccess;
    k_patchify<<<ntiles, 256, 0, stream>>>(pixels, items, cu, tiles, patches, pos, axes);
    return hipGetLastError();
}

// =========================================================== GEMM
//
// C^T tile = W_tile (A operand: rows are output features) x X_tile^T (B
// operand: columns are tokens). Workgroup: BM tokens x BN features, 4 waves in
// 2 x 2, each wave (BM/2) x (BN/2) as (BN/64) x (BM/64) MFMA tiles of 32 x 32.
// K advances in steps of 64 through LDS (one buffer; the next step's global
// loads are in flight in registers while the current step computes). LDS rows
// are 128 bytes; 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so the
// 8 lanes of one ds_read_b128 phase (8 consecutive rows, same chunk) hit 8
// distinct bank groups.

template <int EPI, int TM, int TN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, f32x16 (&acc)[TN][TM], int mw, int nw, int l32,
                                              int hh, const float (&inv)[TM]);

// 1/rms of the folded RMSNorm for token m (1 when the projection reads plain rows):
// the partial sums of squares the row's producer wrote, summed in a fixed order.
__device__ __forceinline__ float folded_inv_rms(const GemmArgs &a, int m) {
    if (!a.ss_in) return 1.f;
    const float *pp = a.ss_in + (size_t)m * kSsParts;
    float ss = 0.f;
    for (int i = 0; i < a.ss_parts; ++i) ss += pp[i];
    return 1.0f / sqrtf(ss / (float)a.K + a.eps);
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
    constexpr int BK = 64;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int WCH = BN * 8 / 256, XCH = BM * 8 / 256;
    __shared__ __attribute__((aligned(16))) u32x4 smem[(BM + BN) * 8];
    u32x4 *sW = smem, *sX = smem + BN * 8;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, hh = lane >> 5;
    const int NT = a.N / BN;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = logical / NT, nt = logical % NT;
    const int m0 = mt * BM, n0 = nt * BN;
    const int K = a.K;

    u32x4 rw[WCH], rx[XCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
            rw[i] = *(const u32x4 *)(a.w + (size_t)(n0 + row) * K + k0 + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
            rx[i] = *(const u32x4 *)(a.x + (size_t)(m0 + row) * K + k0 + ch * 8);
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
            sW[row * 8 + (ch ^ (row & 7))] = rw[i];
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, ch = idx & 7;
            sX[row * 8 + (ch ^ (row & 7))] = rx[i];
        }
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

    gload(0);
    for (int k0 = 0; k0 < K; k0 += BK) {
        sstore();
        __syncthreads();
        if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + hh;
            bf16x8 af[TN], bfr[TM];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int row = wn * WN + tn * 32 + l32;
                af[tn] = __builtin_bit_cast(bf16x8, sW[row * 8 + (ch ^ (row & 7))]);
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int row = wm * WM + tm * 32 + l32;
                bfr[tm] = __builtin_bit_cast(bf16x8, sX[row * 8 + (ch ^ (row & 7))]);
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tn], bfr[tm], acc[tn][tm], 0, 0, 0);
        }
        __syncthreads();
    }

    float inv[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
        inv[tm] = (EPI == kEpiQkv || EPI == kEpiSwiglu) ? folded_inv_rms(a, m0 + wm * WM + tm * 32 + l32) : 1.f;
    gemm_epilogue<EPI, TM, TN>(a, acc, m0 + wm * WM, n0 + wn * WN, l32, hh, inv);
}

// Epilogue of one wave's (TN x TM) grid of 32 x 32 accumulator tiles. The wave's
// features start at nw (a multiple of 64; the wave covers 64 of them), its tokens
// at mw; accumulator register 4i + j of tile (tn, tm) is feature
// nw + 32 tn + 8 i + 4 (lane / 32) + j, token mw + 32 tm + lane % 32.
//
// Folded RMSNorm: a consumer of normalised rows (QKV, gate/up) reads x's bf16 copy
// with the gain already in its weights, and scales its accumulator by 1/rms(x),
// rms from the partial sums of squares the row's producer wrote (one per 64
// features, summed here in a fixed order).
template <int EPI, int TM, int TN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, f32x16 (&acc)[TN][TM], int mw, int nw, int l32,
                                              int hh, const float (&inv)[TM]) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int m = mw + tm * 32 + l32;
        if (m >= a.M) continue;
        if constexpr (EPI == kEpiQkv || EPI == kEpiSwiglu) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) acc[tn][tm] *= inv[tm];
        }
        if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
                const int col0 = nw / 2 + p * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float g = acc[2 * p][tm][i * 4 + j], u = acc[2 * p + 1][tm][i * 4 + j];
                        o[j] = g / (1.0f + __expf(-g)) * u;
                    }
                    const int col = col0 + i * 8 + hh * 4;
                    *(u32x2 *)(a.out_bf16 + (size_t)m * a.ld_out + col) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                }
            }
        } else {
            float ssp = 0.f;  // sum of squares of this wave's 64 output features (residual / patch)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int nbase = nw + tn * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = nbase + i * 8 + hh * 4;
                    float o[4] = {acc[tn][tm][i * 4 + 0], acc[tn][tm][i * 4 + 1], acc[tn][tm][i * 4 + 2],
                                  acc[tn][tm][i * 4 + 3]};
                    if constexpr (EPI == kEpiStore) {
                        *(u32x2 *)(a.out_bf16 + (size_t)m * a.ld_out + n) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                    } else if constexpr (EPI == kEpiResid || EPI == kEpiPatch) {
                        f32x4 *px = (f32x4 *)(a.out_f32 + (size_t)m * a.ld_f32 + n);
                        f32x4 xv;
                        if constexpr (EPI == kEpiResid) {
                            xv = a.res_in ? *(const f32x4 *)(a.res_in + (size_t)m * a.ld_f32 + n) : *px;
                            xv = f32x4{xv.x + o[0], xv.y + o[1], xv.z + o[2], xv.w + o[3]};
                        } else {
                            xv = f32x4{o[0] * a.scale, o[1] * a.scale, o[2] * a.scale, o[3] * a.scale};
                        }
                        *px = xv;
                        if (a.ss_out) {
                            ssp += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
                            *(u32x2 *)(a.out_bf16 + (size_t)m * a.ld_out + n) = u32x2{pack2(xv.x, xv.y), pack2(xv.z, xv.w)};
                        }
                    } else if constexpr (EPI == kEpiQkv) {
                        if (nbase < 2 * a.D) {
                            // rotary: pairs (e, e+1) and (e+2, e+3), e = n % 64 even
                            const u32x2 pw = *(const u32x2 *)(a.pos + (size_t)m * 4);
                            const int p0 = (int)(int16_t)(pw.x & 0xffff), p1 = (int)(int16_t)(pw.x >> 16),
                                      p2 = (int)(int16_t)(pw.y & 0xffff);
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const int pair = ((n & 63) >> 1) + q;
                                const int pv = pair < a.sec0 ? p0 : (pair < a.sec0 + a.sec1 ? p1 : p2);
                                const float2 cs = a.rope[pv * 32 + pair];
                                const float x0 = o[2 * q], x1 = o[2 * q + 1];
                                o[2 * q] = x0 * cs.x - x1 * cs.y;
                                o[2 * q + 1] = x0 * cs.y + x1 * cs.x;
                            }
                            *(u32x2 *)(a.out_bf16 + (size_t)m * a.ld_out + n) =
                                u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                        } else {
                            const int e = n - 2 * a.D;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                a.vt[(size_t)(e + j) * a.ld_vt + m] = (uint16_t)f32_to_bf16(o[j]);
                        }
                    }
                }
            }
            if constexpr (EPI == kEpiResid || EPI == kEpiPatch) {
                if (a.ss_out) {
                    ssp += __shfl_xor(ssp, 32, 64);  // lanes l and l ^ 32 hold the same token
                    if (hh == 0) a.ss_out[(size_t)m * kSsParts + (nw >> 6)] = ssp;
                }
            }
        }
    }
}

// 256 x 256 tiles for N % 256 == 0: 8 waves (2 token rows x 4 feature columns
// of 128 x 64), two LDS stages of 64 KB filled by global_load_lds_dwordx4
// (16 bytes per lane straight into LDS, no register staging). Lane i of a load
// instruction lands at LDS chunk (base + i); the global chunk it fetches is the
// logical chunk that the swizzle assigns to that LDS slot.

typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS of the 256 x 256 kernel (bytes): the two operand stages [0, 128 KB) during
// the K loop; afterwards the epilogue's staging area [0, kStageBytes) and, past
// it, one float per tile token (row scale of the feature-major v tiles).
constexpr int kQkPitch = 528;                 // bf16 rows of 256 values + 16 B
constexpr int kGluPitch = 272;                // bf16 rows of 128 values + 16 B
constexpr int kResPitch = 1040;               // fp32 rows of 256 values + 16 B
constexpr int kResSlice = 64 * kResPitch;     // 64 tokens
constexpr int kStageBytes = 256 * kQkPitch;   // 135,168 >= 2 * kResSlice
constexpr int kSmemBytes = kStageBytes + 256 * 4;
// QKV epilogue: the tile's rotary table rows (256 B of (cos, sin) pairs per token) fill
// one 64 KB operand stage buffer; the other holds one staging area per wave of 32 rows
// of 64 bf16 features.
constexpr int kStageBytes2 = 65536;                    // one operand stage of the K loop
constexpr int kQkStagePitch = 144;                     // 128 B + 16 B
constexpr int kQkStageBytes = 32 * kQkStagePitch;      // 4,608 per wave
static_assert(256 * 256 <= kStageBytes2 && 8 * kQkStageBytes <= kStageBytes2, "QKV epilogue LDS");

// K loop of one tile. SWAP = false: MFMA A operand = weight rows, B = token
// rows, so lane (l32, hh) holds features 8 i + 4 hh + j of token l32 in register
// 4 i + j. SWAP = true (feature-major v tiles): A = token rows, so the lane holds
// tokens 8 i + 4 hh + j of feature l32.
// `before_last(buffer)` runs right before the last stage's products, once the other stage buffer is free
// (its last reads retired at the preceding barrier, and no DMA targets it any more); it may start DMA into
// that buffer, which the epilogue then waits for.
template <bool FP8, bool SWAP, typename BeforeLast>
__device__ __forceinline__ void gemm256_kloop(const GemmArgs &a, u32x4 *smem, f32x16 (&acc)[2][4], int m0, int n0,
                                              int wave, int lane, BeforeLast &&before_last) {
    constexpr int BM = 256, BN = 256, ES = FP8 ? 1 : 2, BK = 128 / ES;
    constexpr int STAGE = (BM + BN) * 8;  // 16-byte chunks per stage
    const int wm = wave & 1, wn = wave >> 1, l32 = lane & 31, hh = lane >> 5;
    const size_t row_bytes = (size_t)a.K * ES;
    const uint8_t *wb = (const uint8_t *)a.w, *xb = (const uint8_t *)a.x;
    // load round r (0..3 weights, 4..7 activations): chunk slot 512 r + 64 wave + lane
    // of the operand tile, row (64 r + slot / 8), LDS chunk slot % 8
    const int prow = (wave * 64 + lane) >> 3, pch = lane & 7;
    auto issue = [&](int k0, int buf) {
        u32x4 *dst = smem + buf * STAGE;
        const size_t kb = (size_t)k0 * ES;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r * 64 + prow;
            lds_dma16(wb + (size_t)(n0 + row) * row_bytes + kb + swz(row, pch) * 16, dst + r * 512 + wave * 64);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r * 64 + prow;
            lds_dma16(xb + (size_t)(m0 + row) * row_bytes + kb + swz(row, pch) * 16,
                      dst + BN * 8 + r * 512 + wave * 64);
        }
    };
    auto mfma = [&](const auto &w_op, const auto &x_op, f32x16 &c) {
        if constexpr (FP8) {
            // v_mfma_scale_f32_32x32x64_f8f6f4, both operands OCP E4M3 (format 0),
            // unit E8M0 block scales (127)
            if constexpr (SWAP)
                c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x_op, w_op, c, 0, 0, 0, 127, 0, 127);
            else
                c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w_op, x_op, c, 0, 0, 0, 127, 0, 127);
        } else {
            if constexpr (SWAP)
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x_op, w_op, c, 0, 0, 0);
            else
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w_op, x_op, c, 0, 0, 0);
        }
    };
    auto compute = [&](const u32x4 *sW) {
        const u32x4 *sX = sW + BN * 8;
        if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int ch = ks * 2 + hh;  // lane half hh supplies 8 consecutive k
                bf16x8 af[2], bfr[4];
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const int row = wn * 64 + tn * 32 + l32;
                    af[tn] = __builtin_bit_cast(bf16x8, sW[row * 8 + swz(row, ch)]);
                }
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const int row = wm * 128 + tm * 32 + l32;
                    bfr[tm] = __builtin_bit_cast(bf16x8, sX[row * 8 + swz(row, ch)]);
                }
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int tm = 0; tm < 4; ++tm) mfma(af[tn], bfr[tm], acc[tn][tm]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = ks * 4 + hh * 2;  // lane half hh supplies 32 consecutive k bytes
                i32x8 af[2], bfr[4];
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const int row = wn * 64 + tn * 32 + l32;
                    const u32x4 lo = sW[row * 8 + swz(row, ch)], hi = sW[row * 8 + swz(row, ch + 1)];
                    af[tn] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const int row = wm * 128 + tm * 32 + l32;
                    const u32x4 lo = sX[row * 8 + swz(row, ch)], hi = sX[row * 8 + swz(row, ch + 1)];
                    bfr[tm] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int tm = 0; tm < 4; ++tm) mfma(af[tn], bfr[tm], acc[tn][tm]);
            }
        }
    };
    // One stage: wait for this wave's DMA of the stage (the next stage's 8 loads
    // may stay in flight), barrier so every wave's DMA is visible, compute, then
    // drain LDS reads and barrier again before the buffer is refilled. Plain
    // s_barrier: a __syncthreads() fence would also wait for the next stage.
    const int nk = a.K / BK;
    issue(0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
        if (kt + 1 < nk) {
            issue((kt + 1) * BK, 1);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        lds_barrier();
        if (kt == nk - 1 && nk >= 2) before_last(1);
        compute(smem);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        if (kt + 1 < nk) {
            if (kt + 2 < nk) {
                issue((kt + 2) * BK, 0);
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            lds_barrier();
            if (kt + 1 == nk - 1) before_last(0);
            compute(smem + STAGE);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
        }
    }
}

// Rotary on four consecutive features (pairs (e, e+1), (e+2, e+3), e = feature
// % 64 even) of one token: cs holds the two (cos, sin) entries.
__device__ __forceinline__ void rotate4(float (&o)[4], const float2 (&cs)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float x0 = o[2 * q], x1 = o[2 * q + 1];
        o[2 * q] = x0 * cs[q].x - x1 * cs[q].y;
        o[2 * q + 1] = x0 * cs[q].y + x1 * cs[q].x;
    }
}

// Epilogues of the 256 x 256 kernel, all staged through LDS so that every global
// access of a wave instruction covers whole rows with 16 bytes per lane: 512 B
// bf16 rows (q, k, plain store, feature-major v), 256 B rows (SwiGLU output) or
// 1 KB fp32 rows (residual and patch, with the bf16 copy and the row's sum of
// squares over the tile's 256 features).
template <int EPI, bool FP8>
__global__ __launch_bounds__(512, 1) void k_gemm256(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) u32x4 smem[kSmemBytes / 16];
    uint8_t *L = (uint8_t *)smem;
    float *row_scale = (float *)(L + kStageBytes);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, hh = lane >> 5;
    const int NT = a.N / 256;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (logical / NT) * 256, n0 = (logical % NT) * 256;
    const bool vtile = EPI == kEpiQkv && n0 >= 2 * a.D;

    // per-token epilogue inputs, loaded before the K loop so their latency hides
    // behind it (and only used after it): the partial sums of squares of the
    // folded RMSNorm (up to 4 parts here; more are read in the epilogue) and the
    // rotary coordinates
    constexpr bool kNorm = EPI == kEpiQkv || EPI == kEpiSwiglu;
    const bool ss_early = kNorm && a.ss_in && a.ss_parts <= 4;
    f32x4 ssv[4] = {};
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int m = m0 + wm * 128 + tm * 32 + l32;
        if (ss_early) ssv[tm] = *(const f32x4 *)(a.ss_in + (size_t)m * kSsParts);
    }
    // coordinates of the tokens whose rotary rows this wave fetches (128 wm + 32 wn + l32); rows past M
    // hold whatever an earlier call left in the arena, so they take coordinate 0 and never index the table
    u32x2 mine = {};
    if constexpr (EPI == kEpiQkv) {
        const int m = m0 + wm * 128 + wn * 32 + l32;
        if (m < a.M) mine = *(const u32x2 *)(a.pos + (size_t)m * 4);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // QKV q/k tiles: the tile's rotary table rows (32 (cos, sin) pairs per token, each pair from the row of
    // its axis' coordinate, 256 B) enter LDS by DMA during the last K stage, into the stage buffer that stage
    // does not read (16-byte DMAs, or 4-byte ones where an axis section has odd length); wave (wm, wn)
    // fetches tokens 128 wm + 32 wn .. + 31,
    // whose coordinates its lanes loaded above (tm = wn). The 16-byte chunk c of token t's row is stored at
    // chunk c ^ (t % 16), so 16 lanes reading the same chunk of 16 consecutive rows cover all 64 banks.
    int rope_buf = -1;
    auto fetch_rope = [&](int buf) {
        if constexpr (EPI == kEpiQkv) {
            rope_buf = buf;
            uint8_t *dst = L + buf * kStageBytes2 + (wm * 128 + wn * 32) * 256;
            const uint8_t *rope = (const uint8_t *)a.rope;
            // (rolled loops: unrolled, the compiler keeps every lane offset live through the K loop)
            if (a.sec0 >= 32 || ((a.sec0 | a.sec1) & 1) == 0) {
                // every 16-byte chunk (two pairs) lies within one axis' section: one 16-byte DMA per lane,
                // four tokens per instruction; lane l fetches stored chunk l % 16 of token 4 it + l / 16,
                // whose coordinate sits in lane (token) of the wave
#pragma unroll 1
                for (int it = 0; it < 8; ++it) {
                    const int r = it * 4 + (lane >> 4);
                    const int c = (lane & 15) ^ (r & 15);  // chunk of the table row: pairs 2 c, 2 c + 1
                    const uint32_t px = (uint32_t)__shfl((int)mine.x, r, 64);
                    const uint32_t py = (uint32_t)__shfl((int)mine.y, r, 64);
                    const int p = 2 * c < a.sec0 ? (int)(int16_t)(px & 0xffff)
                                                 : (2 * c < a.sec0 + a.sec1 ? (int)(int16_t)(px >> 16)
                                                                            : (int)(int16_t)(py & 0xffff));
                    lds_dma16(rope + p * 256 + c * 16, dst + it * 1024);
                }
            } else {  // a section of odd length: pairs of one chunk may take different rows, one dword each
#pragma unroll 1
                for (int r = 0; r < 32; ++r) {
                    const int gd = (((lane >> 2) ^ (r & 15)) << 2) | (lane & 3);
                    const int pair = gd >> 1;
                    const uint32_t px = (uint32_t)__builtin_amdgcn_readlane((int)mine.x, r);
                    const uint32_t py = (uint32_t)__builtin_amdgcn_readlane((int)mine.y, r);
                    const int p = pair < a.sec0 ? (int)(int16_t)(px & 0xffff)
                                                : (pair < a.sec0 + a.sec1 ? (int)(int16_t)(px >> 16)
                                                                          : (int)(int16_t)(py & 0xffff));
                    lds_dma4(rope + p * 256 + gd * 4, dst + r * 256);
                }
            }
        }
    };
    if (vtile)
        gemm256_kloop<FP8, true>(a, smem, acc, m0, n0, wave, lane, [](int) {});
    else
        gemm256_kloop<FP8, false>(a, smem, acc, m0, n0, wave, lane, fetch_rope);

    // per-token row factor of lane token (m0 + 128 wm + 32 tm + l32): folded
    // RMSNorm 1/rms (fixed summation order: part 0, 1, 2, ...) times the E4M3
    // activation scale
    float fac[4] = {1.f, 1.f, 1.f, 1.f};
    const float inv_k = 1.0f / (float)a.K;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int m = m0 + wm * 128 + tm * 32 + l32;
        if (kNorm && a.ss_in) {
            if (ss_early) {
                float ss = ssv[tm].x;
                if (a.ss_parts > 1) ss += ssv[tm].y;
                if (a.ss_parts > 2) ss += ssv[tm].z;
                if (a.ss_parts > 3) ss += ssv[tm].w;
                fac[tm] = __builtin_amdgcn_rsqf(ss * inv_k + a.eps);
            } else {
                fac[tm] = folded_inv_rms(a, m);
            }
        }
        if constexpr (FP8) fac[tm] *= a.x_scale[m];
    }

    if constexpr (EPI == kEpiQkv) {
        if (vtile) {
            // ---- feature-major v: rows = 256 features of the tile, 512 B of tokens each
            if (wn == 0 && hh == 0) {
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) row_scale[wm * 128 + tm * 32 + l32] = fac[tm];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
            const float wsc = FP8 ? a.w_scale : 1.0f;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const int f = wn * 64 + tn * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = wm * 128 + tm * 32 + i * 8 + hh * 4;
                        const f32x4 s = *(const f32x4 *)(row_scale + t);
                        f32x4 v = {acc[tn][tm][i * 4], acc[tn][tm][i * 4 + 1], acc[tn][tm][i * 4 + 2],
                                   acc[tn][tm][i * 4 + 3]};
                        v *= s;
                        if constexpr (FP8) v *= wsc;
                        *(u32x2 *)(L + f * kQkPitch + t * 2) = u32x2{pack2(v.x, v.y), pack2(v.z, v.w)};
                    }
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
            // tokens past M are written as zeros (masked keys must hold finite values)
            const bool full = m0 + 256 <= a.M;
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int f = it * 16 + wave * 2 + hh, t0 = l32 * 8;
                u32x4 v = *(const u32x4 *)(L + f * kQkPitch + t0 * 2);
                const int valid = a.M - (m0 + t0);
                if (!full && valid < 8) {
                    uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = 2 * e < valid ? 0xffffu : 0u, hi = 2 * e + 1 < valid ? 0xffff0000u : 0u;
                        w4[e] &= lo | hi;
                    }
                    v = u32x4{w4[0], w4[1], w4[2], w4[3]};
                }
                __builtin_nontemporal_store(v, (u32x4 *)(a.vt + (size_t)(n0 - 2 * a.D + f) * a.ld_vt + m0 + t0));
            }
            return;
        }
    }

    if constexpr (EPI == kEpiQkv) {
        // ---- rotated q, k rows: every wave rotates its 128 tokens x 64 features with the table rows the K
        // loop fetched (a K of one stage fetches them here), and stores them through a wave-private staging
        // area in the other stage buffer, 32 tokens at a time, as whole 128-byte row segments.
        if (rope_buf < 0) fetch_rope(1);
        wait_vmcnt<0>();
        lds_barrier();
        const float wsc = FP8 ? a.w_scale : 1.0f;
        const uint8_t *rope_lds = L + rope_buf * kStageBytes2;
        uint8_t *stage = L + (1 - rope_buf) * kStageBytes2 + wave * kQkStageBytes;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int t = wm * 128 + tm * 32 + l32;
            const float k = fac[tm] * wsc;
            const uint8_t *row = rope_lds + t * 256;
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cl = tn * 32 + i * 8 + hh * 4;  // feature within the wave's 64
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = acc[tn][tm][i * 4 + j] * k;
                    // pairs 2 hh, 2 hh + 1 of the group of 4 starting at pair 16 tn + 4 i: chunk 8 tn + 2 i + hh
                    const f32x4 e = *(const f32x4 *)(row + (((tn * 8 + i * 2 + hh) ^ (t & 15)) << 4));
                    const float2 cs[2] = {float2{e.x, e.y}, float2{e.z, e.w}};
                    rotate4(o, cs);
                    *(u32x2 *)(stage + l32 * kQkStagePitch + cl * 2) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int chunk = it * 64 + lane, r = chunk >> 3, part = chunk & 7;
                const int m = m0 + wm * 128 + tm * 32 + r;
                const u32x4 v = *(const u32x4 *)(stage + r * kQkStagePitch + part * 16);
                if (m < a.M)
                    __builtin_nontemporal_store(v, (u32x4 *)(a.out_bf16 + (size_t)m * a.ld_out + n0 + wn * 64 + part * 8));
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // staging read back before the next tm writes it
        }
    } else if constexpr (EPI == kEpiStore) {
        // ---- token-major bf16 rows of 256 features
        const float wsc = FP8 ? a.w_scale : 1.0f;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int t = wm * 128 + tm * 32 + l32;
            const float k = fac[tm] * wsc;
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = wn * 64 + tn * 32 + i * 8 + hh * 4;
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = acc[tn][tm][i * 4 + j] * k;
                    *(u32x2 *)(L + t * kQkPitch + c * 2) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int t = it * 16 + wave * 2 + hh, m = m0 + t;
            const u32x4 v = *(const u32x4 *)(L + t * kQkPitch + l32 * 16);
            if (m < a.M) __builtin_nontemporal_store(v, (u32x4 *)(a.out_bf16 + (size_t)m * a.ld_out + n0 + l32 * 8));
        }
    } else if constexpr (EPI == kEpiSwiglu) {
        // ---- gate (tn 0) and up (tn 1) of 32 outputs per wave: output column
        // 32 wn + 8 i + 4 hh + j of the tile's 128; rows of 256 B
        const float sg = FP8 ? a.w_scale : 1.0f, su = FP8 ? a.w_scale2 : 1.0f;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int t = wm * 128 + tm * 32 + l32;
            // g = ag kg, u = au ku: SiLU(g) u = ag au (kg ku) / (1 + 2^(ag (-kg log2 e)))
            const float kg = fac[tm] * sg, ke = kg * -1.4426950408889634f, kgu = kg * fac[tm] * su;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float ag = acc[0][tm][i * 4 + j], au = acc[1][tm][i * 4 + j];
                    const float e = __builtin_amdgcn_exp2f(ag * ke);
                    o[j] = ag * au * kgu * __builtin_amdgcn_rcpf(1.0f + e);
                }
                *(u32x2 *)(L + t * kGluPitch + (wn * 32 + i * 8 + hh * 4) * 2) =
                    u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int t = it * 32 + wave * 4 + (lane >> 4), m = m0 + t, ch = lane & 15;
            const u32x4 v = *(const u32x4 *)(L + t * kGluPitch + ch * 16);
            if (m < a.M) __builtin_nontemporal_store(v, (u32x4 *)(a.out_bf16 + (size_t)m * a.ld_out + n0 / 2 + ch * 8));
        }
        if (a.gu_out) {
            // the pre-activations themselves (g, u in the interleaved column order of the product), for
            // a backward pass: 512-byte rows through LDS like the plain store
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const int t = wm * 128 + tm * 32 + l32;
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const float k = fac[tm] * (tn ? su : sg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = wn * 64 + tn * 32 + i * 8 + hh * 4;
                        *(u32x2 *)(L + t * kQkPitch + c * 2) =
                            u32x2{pack2(acc[tn][tm][i * 4] * k, acc[tn][tm][i * 4 + 1] * k),
                                  pack2(acc[tn][tm][i * 4 + 2] * k, acc[tn][tm][i * 4 + 3] * k)};
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int t = it * 16 + wave * 2 + hh, m = m0 + t;
                const u32x4 v = *(const u32x4 *)(L + t * kQkPitch + l32 * 16);
                if (m < a.M) __builtin_nontemporal_store(v, (u32x4 *)(a.gu_out + (size_t)m * a.ld_gu + n0 + l32 * 8));
            }
        }
    } else {
        // ---- residual / patch: four slices of 64 tokens (slice s = tile tokens
        // [64 s, 64 s + 64), held by the waves with wm = s / 2 at tm = 2 (s % 2) +
        // 0, 1), double-buffered in LDS; wave w finishes rows 8 w .. 8 w + 7 of a
        // slice: x (fp32, read one slice ahead) += acc, its bf16 copy, and the sum
        // of squares of the row's 256 new values
        const float wsc = FP8 ? a.w_scale : 1.0f;
        f32x4 xin[2][8];
        auto load_x = [&](int s, f32x4 (&dst)[8]) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int m = m0 + s * 64 + wave * 8 + k;
                dst[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (EPI == kEpiResid && m < a.M)
                    dst[k] = *(const f32x4 *)((a.res_in ? a.res_in : a.out_f32) + (size_t)m * a.ld_f32 + n0 + lane * 4);
            }
        };
        load_x(0, xin[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float *S = (float *)(L + (s & 1) * kResSlice);
            if (wm == (s >> 1)) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int tm = 2 * (s & 1) + q, r = q * 32 + l32;
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = wn * 64 + tn * 32 + i * 8 + hh * 4;
                            f32x4 v = {acc[tn][tm][i * 4], acc[tn][tm][i * 4 + 1], acc[tn][tm][i * 4 + 2],
                                       acc[tn][tm][i * 4 + 3]};
                            if constexpr (FP8) v *= fac[tm] * wsc;
                            *(f32x4 *)((uint8_t *)S + r * kResPitch + c * 4) = v;
                        }
                }
            }
            if (s + 1 < 4) load_x(s + 1, xin[(s + 1) & 1]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            lds_barrier();
            float sq[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = wave * 8 + k, m = m0 + s * 64 + r;
                const f32x4 d = *(const f32x4 *)((const uint8_t *)S + r * kResPitch + lane * 16);
                const f32x4 v = EPI == kEpiResid ? xin[s & 1][k] + d : d * a.scale;
                sq[k] = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                if (m < a.M) {
                    __builtin_nontemporal_store(v, (f32x4 *)(a.out_f32 + (size_t)m * a.ld_f32 + n0 + lane * 4));
                    if (a.ss_out)
                        __builtin_nontemporal_store(u32x2{pack2(v.x, v.y), pack2(v.z, v.w)},
                                                    (u32x2 *)(a.out_bf16 + (size_t)m * a.ld_out + n0 + lane * 4));
                }
            }
            if (a.ss_out) {
                // row sums over the 64 lanes for all 8 rows at once: each exchange step
                // halves the rows a lane keeps (lane bits 5, 4, 3 pick them), the last
                // three finish the sum; lane 8 b then holds row b
                const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
                float s4[4], s2[2];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s4[j] = (b5 ? sq[4 + j] : sq[j]) + __shfl_xor(b5 ? sq[j] : sq[4 + j], 32, 64);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    s2[j] = (b4 ? s4[2 + j] : s4[j]) + __shfl_xor(b4 ? s4[j] : s4[2 + j], 16, 64);
                float s1 = (b3 ? s2[1] : s2[0]) + __shfl_xor(b3 ? s2[0] : s2[1], 8, 64);
                s1 += __shfl_xor(s1, 4, 64);
                s1 += __shfl_xor(s1, 2, 64);
                s1 += __shfl_xor(s1, 1, 64);
                const int m = m0 + s * 64 + wave * 8 + (lane >> 3);
                if ((lane & 7) == 0 && m < a.M) a.ss_out[(size_t)m * kSsParts + (n0 >> 8)] = s1;
            }
        }
    }
}

template <int BM, int BN>
static hipError_t gemm_dispatch(int epi, const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * (a.N / BN);
    switch (epi) {
        case kEpiStore: k_gemm<BM, BN, kEpiStore><<<tiles, 256, 0, stream>>>(a); break;
        case kEpiQkv: k_gemm<BM, BN, kEpiQkv><<<tiles, 256, 0, stream>>>(a); break;
        case kEpiResid: k_gemm<BM, BN, kEpiResid><<<tiles, 256, 0, stream>>>(a); break;
        case kEpiSwiglu: k_gemm<BM, BN, kEpiSwiglu><<<tiles, 256, 0, stream>>>(a); break;
        case kEpiPatch: k_gemm<BM, BN, kEpiPatch><<<tiles, 256, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool FP8>
static hipError_t gemm256_dispatch(int epi, const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.M + 255) / 256) * (a.N / 256);
    switch (epi) {
        case kEpiStore: k_gemm256<kEpiStore, FP8><<<tiles, 512, 0, stream>>>(a); break;
        case kEpiQkv: k_gemm256<kEpiQkv, FP8><<<tiles, 512, 0, stream>>>(a); break;
        case kEpiResid: k_gemm256<kEpiResid, FP8><<<tiles, 512, 0, stream>>>(a); break;
        case kEpiSwiglu: k_gemm256<kEpiSwiglu, FP8><<<tiles, 512, 0, stream>>>(a); break;
        case kEpiPatch: k_gemm256<kEpiPatch, FP8><<<tiles, 512, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmArgs &a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    if (a.N % 128 != 0 || a.K % 64 != 0) return hipErrorInvalidValue;
    if (a.N % 256 == 0) return gemm256_dispatch<false>(epi, a, stream);
    if (a.gu_out) return hipErrorInvalidValue;  // only the 256-column tiles store pre-activations
    return gemm_dispatch<256, 128>(epi, a, stream);
}

hipError_t launch_gemm_e4m3(int epi, const GemmArgs &a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    if (a.N % 256 != 0 || a.K % 128 != 0 || !a.x_scale) return hipErrorInvalidValue;
    return gemm256_dispatch<true>(epi, a, stream);
}

// =========================================================== attention
//
// Bidirectional attention inside each item (varlen, tiles from the tape's
// prefix sums). Workgroup = (query tile of 256 tokens of one item, head), 8
// waves of 32 queries; key tiles of 64 keys staged in LDS by DMA in four
// buffers taken a pair of tiles at a time, one barrier per pair (the next pair
// loads while this one is computed). Per key tile:
//   S^T (keys x queries) = K Q^T   -- each lane keeps one query and 32 of its
//                                      scores; the row max needs one exchange
//                                      between the two lane halves
//   online softmax in fp32 on exp2 of pre-scaled logits: the score accumulators
//   start at minus a per-query reference (the first tile's max), so a weight
//   costs one exponential; the reference moves up, rescaling the output, only
//   when a tile's weights of some query sum past 2^8, so most tiles take no max
//   O^T (d x queries) += V^T P^T   -- P^T comes straight from the S^T registers.
// Small waves (under 128 registers) let four waves share each SIMD, so the
// softmax of some waves runs on the vector ALUs while others keep the matrix
// cores busy.
// Within each 32-key subtile, LDS row r of K holds key perm32(r), chosen so that
// the 8 scores a lane feeds to one PV step belong to 8 consecutive keys; V^T rows
// (feature-major vt) are then read as one 16-byte chunk, like K. Both operands
// use 16-byte chunks XOR-swizzled by (row / 2) % 8: conflict-free ds_read_b128
// on 64 banks.

__device__ __forceinline__ int perm32(int r) {  // r = 8 i + 4 h + j
    const int i = r >> 3, h = (r >> 2) & 1, j = r & 3;
    return (i >> 1) * 16 + h * 8 + (i & 1) * 4 + j;
}

constexpr float kRescaleSum = 256.0f;  // attention: largest sum of one query's weights in a tile half

__global__ __launch_bounds__(512, 2) void k_attention(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                      int ldqk, const uint16_t *__restrict__ vt, int ldvt,
                                                      uint16_t *__restrict__ o, int ldo, const int *__restrict__ cu,
                                                      const int2 *__restrict__ tiles, int ntiles,
                                                      float *__restrict__ lse, int ldl) {
    constexpr int NS = 4;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int head = logical / ntiles, ti = logical % ntiles;
    const int2 tile = tiles[ti];
    const int k0 = cu[tile.x], k1 = cu[tile.x + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    constexpr int STAGE = 1024;  // 16-byte chunks: K tile 512 | V^T tile 512
    __shared__ __attribute__((aligned(1024))) u32x4 smem[NS * STAGE];

    const int qbase = tile.y + wave * 32;
    const bool active = qbase < k1;
    const bool qvalid = qbase + l32 < k1;
    // queries pre-scaled by c = log2(e) / sqrt(64): scores come out of the MFMAs in
    // base-2 logit units
    const float c = 0.18033688011112042f;
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 raw = __builtin_bit_cast(
            bf16x8, *(const u32x4 *)(q + (size_t)(qbase + l32) * ldqk + head * 64 + ks * 16 + hh * 8));
        qf[ks] = __builtin_convertvector(__builtin_convertvector(raw, f32x8) * c, bf16x8);
    }

    // DMA of stage t into buffer t % NS: thread tid moves K chunk slot tid and V^T
    // chunk slot tid (row slot / 8, stored chunk slot % 8)
    const int prow = tid >> 3, pc = swz(prow, tid & 7);
    const int pkey = (prow & 32) + perm32(prow & 31);
    auto issue = [&](int t) {
        const int kt = k0 + t * 64;
        u32x4 *dst = smem + (t % NS) * STAGE;
        lds_dma16(k + (size_t)(kt + pkey) * ldqk + head * 64 + pc * 8, dst + wave * 64);
        lds_dma16(vt + (size_t)(head * 64 + prow) * ldvt + kt + pc * 8, dst + 512 + wave * 64);
    };

    f32x16 O[2] = {f32x16{}, f32x16{}};
    float m_run = 0.f, l_run = 0.f;  // reference (running max) of the scaled scores, sum of weights

    auto compute = [&](const u32x4 *sK, int kt, bool first) {
        const u32x4 *sV = sK + 512;
        // the accumulators start at -m_run: the MFMAs return scores relative to the
        // reference, ready for the exponential
        f32x16 S[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int row = kk * 32 + l32;
            S[kk] = -m_run;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, sK[row * 8 + swz(row, ks * 2 + hh)]);
                S[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[kk], 0, 0, 0);
            }
        }
        if (kt + 64 > k1) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt + kk * 32 + perm32((r >> 2) * 8 + hh * 4 + (r & 3));
                    if (key >= k1) S[kk][r] = -INFINITY;
                }
        }
        // moves the reference up by the query's largest relative score (never down; the first tile
        // sets it) and rescales what was summed so far
        auto rebase = [&]() {
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kk][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float d = first ? mx : fmaxf(mx, 0.f);
            m_run += d;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) S[kk] -= d;
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(-d);
                l_run *= alpha;
                O[0] *= alpha;
                O[1] *= alpha;
            }
        };
        // p = 2^(relative score) on the raw v_exp_f32 (weights below 2^-126 flush to
        // 0); packed to bf16 at once, and the row sum taken over those same bf16 values
        u32x4 P[2][2];
        float rs = 0.f;
        auto weights = [&]() {
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            rs = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = ip * 4 + e;
                        const float p0 = __builtin_amdgcn_exp2f(S[kk][2 * r]);
                        const float p1 = __builtin_amdgcn_exp2f(S[kk][2 * r + 1]);
                        const bf16x2 pb = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
                        w[e] = __builtin_bit_cast(uint32_t, pb);
                        rs = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, rs, false);
                    }
                    P[kk][ip] = u32x4{w[0], w[1], w[2], w[3]};
                }
        };
        // Later tiles keep the reference unless some query's weights in the tile sum past 2^8 (so
        // every weight is at most 2^8, which the bf16 weights and fp32 sums hold as well as weights
        // up to 1; a sum that overflowed or is NaN fails the test too): then the reference moves
        // and the weights are taken again. The softmax does not depend on the reference, most
        // tiles keep it, and they need no maximum. Only queries inside the item vote: the lanes
        // past its end hold whatever rows follow it, and must not change the reference of the
        // others, or a row would depend on its batch.
        if (first) rebase();
        weights();
        if (!first && __any(qvalid && !(rs <= kRescaleSum))) {
            rebase();
            weights();
        }
        l_run += rs;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int kk = s2 >> 1, ip = s2 & 1;
            const bf16x8 pf = __builtin_bit_cast(bf16x8, P[kk][ip]);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int row = dt * 32 + l32;
                const bf16x8 vf = __builtin_bit_cast(bf16x8, sV[row * 8 + swz(row, kk * 4 + ip * 2 + hh)]);
                O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, O[dt], 0, 0, 0);
            }
        }
    };

    const int ntile = (k1 - k0 + 63) >> 6;
    // key tiles in pairs, one barrier per pair: the barrier publishes both tiles of the pair and
    // retires every wave's reads of the previous pair, whose two buffers then receive the next pair
    if (0 < ntile) issue(0);
    if (1 < ntile) issue(1);
    for (int t = 0; t < ntile; t += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        if (t + 2 < ntile) issue(t + 2);
        if (t + 3 < ntile) issue(t + 3);
        if (active) {
            compute(smem + (t % NS) * STAGE, k0 + t * 64, t == 0);
            if (t + 1 < ntile) compute(smem + ((t + 1) % NS) * STAGE, k0 + (t + 1) * 64, false);
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const int qrow = qbase + l32;
    if (active && qrow < k1) {
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = dt * 32 + i * 8 + hh * 4;
                *(u32x2 *)(o + (size_t)qrow * ldo + head * 64 + d) =
                    u32x2{pack2(O[dt][i * 4 + 0] * inv, O[dt][i * 4 + 1] * inv),
                          pack2(O[dt][i * 4 + 2] * inv, O[dt][i * 4 + 3] * inv)};
            }
        // log2 of the softmax denominator in the pre-scaled (base-2) logit units, head-major; the
        // backward pass rebuilds the weights from it
        if (lse && hh == 0) lse[(size_t)head * ldl + qrow] = m_run + __log2f(l_tot);
    }
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, int ldqk, const uint16_t *vt, int ldvt,
                            uint16_t *o, int ldo, const int *cu, const int2 *tiles, int ntiles, int heads,
                            hipStream_t stream, float *lse, int ldl) {
    if (ntiles == 0) return hipSuccess;
    k_attention<<<ntiles * heads, 512, 0, stream>>>(q, k, ldqk, vt, ldvt, o, ldo, cu, tiles, ntiles, lse, ldl);
    return hipGetLastError();
}

// =========================================================== MaxSim
//
// Hard MaxSim of every (query item, document item) pair. Workgroup = one
// document and four queries (one per wave): the document's rows pass through
// LDS once, in double-buffered tiles of 32 rows filled by DMA, and all four
// waves score them. Each wave holds its query's counted rows (64 per pass, zero
// past the end) as the MFMA B operand in registers and reads the document tile
// as the A operand (16-byte chunks XOR-swizzled by row % 16: conflict-free).
// Output S^T: a lane holds 16 document rows of one query row, so the running max
// stays in registers; the two lane halves are merged at the end of a pass and
// the wave sums the counted rows. Document rows past the end repeat the last
// row, which cannot change a maximum.
template <int KS>  // columns / 16
__global__ __launch_bounds__(256) void k_maxsim(const uint16_t *__restrict__ q, const size_t *__restrict__ qoff,
                                                size_t qrows, size_t qld, int nq, const uint16_t *__restrict__ d,
                                                const size_t *__restrict__ doff, size_t drows, size_t dld, int nd,
                                                size_t prefix, size_t span, float *__restrict__ scores, size_t ld) {
    constexpr int CH = 2 * KS;        // 16-byte chunks per row
    constexpr int TILE = 32 * CH;     // chunks per tile of 32 rows
    constexpr int LPT = TILE / 256;   // DMA loads per thread per tile
    __shared__ __attribute__((aligned(1024))) u32x4 sD[2 * TILE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int groups = (nq + 3) / 4;
    const int j = blockIdx.x / groups, grp = blockIdx.x % groups;
    // counted rows [qa, qb) of query grp*4 + w; empty past nq
    auto query_rows = [&](int w, size_t &qa, size_t &qb) {
        const int i = grp * 4 + w;
        qa = qb = 0;
        if (i >= nq) return;
        size_t q0 = min(qoff[i], qrows), q1 = max(q0, min(qoff[i + 1], qrows));
        qa = min(q0 + prefix, q1), qb = min(q1, qa + span);
    };
    size_t qa, qb;
    query_rows(wave, qa, qb);
    int passes = 0;  // uniform over the workgroup
    for (int w = 0; w < 4; ++w) {
        size_t a, b;
        query_rows(w, a, b);
        passes = max(passes, (int)((b - a + 63) / 64));
    }
    const size_t d0 = min(doff[j], drows), d1 = max(d0, min(doff[j + 1], drows));
    const int ntiles = (int)((d1 - d0 + 31) / 32);
    float total = 0.f;
    if (ntiles > 0) {
        auto issue = [&](int t, int buf) {
#pragma unroll
            for (int r = 0; r < LPT; ++r) {
                const int p = r * 256 + tid, row = p / CH, c = (p % CH) ^ (row & 15);
                const size_t src = min(d0 + (size_t)t * 32 + row, d1 - 1);
                lds_dma16(d + src * dld + c * 8, sD + buf * TILE + r * 256 + wave * 64);
            }
        };
        for (int pass = 0; pass < passes; ++pass) {
            const size_t c0 = qa + (size_t)pass * 64;
            bf16x8 qf[2][KS];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const size_t r = c0 + b * 32 + l32;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qf[b][ks] = r < qb ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(q + r * qld + ks * 16 + hh * 8))
                                       : bf16x8{};
            }
            float best[2] = {-INFINITY, -INFINITY};
            issue(0, 0);
            for (int t = 0; t < ntiles; ++t) {
                if (t + 1 < ntiles) {
                    issue(t + 1, (t + 1) & 1);
                    if constexpr (LPT == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                lds_barrier();
                const u32x4 *tile = sD + (t & 1) * TILE;
                f32x16 S[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 df = __builtin_bit_cast(bf16x8, tile[l32 * CH + ((ks * 2 + hh) ^ (l32 & 15))]);
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        S[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df, qf[b][ks], S[b], 0, 0, 0);
                }
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 16; ++e) best[b] = fmaxf(best[b], S[b][e]);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                lds_barrier();
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const float m = fmaxf(best[b], __shfl_xor(best[b], 32, 64));
                const size_t r = c0 + b * 32 + l32;
                total += (hh == 0 && r < qb) ? m : 0.f;
            }
        }
        total = qb > qa ? wave_sum(total) / (float)(qb - qa) : 0.f;
    }
    const int i = grp * 4 + wave;
    if (i < nq && lane == 0) scores[(size_t)i * ld + j] = total;
}

hipError_t launch_maxsim(const uint16_t *q, const size_t *qoff, size_t qrows, size_t qld, int nq, const uint16_t *d,
                         const size_t *doff, size_t drows, size_t dld, int nd, int columns, size_t prefix, size_t span,
                         float *scores, size_t ld, hipStream_t stream) {
    if (nq == 0 || nd == 0) return hipSuccess;
    const long blocks_l = (long)((nq + 3) / 4) * nd;
    if (blocks_l > 0x7fffffffL) return hipErrorInvalidValue;
    const int blocks = (int)blocks_l;
    if (columns == 128)
        k_maxsim<8><<<blocks, 256, 0, stream>>>(q, qoff, qrows, qld, nq, d, doff, drows, dld, nd, prefix, span, scores, ld);
    else if (columns == 256)
        k_maxsim<16><<<blocks, 256, 0, stream>>>(q, qoff, qrows, qld, nq, d, doff, drows, dld, nd, prefix, span, scores, ld);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// =========================================================== pool
//
// Scores s[t][h] = xf_t . u_h with u_h = W_k,h q_h / 8 (the reassociated form of
// q_h . (xf_t W_k)_h / sqrt(64)) come from the final norm kernel. Two launches:
//  - token-parallel, one workgroup per 256-token tile of an item (the attention
//    tile list): per head h, m = max over the tile's tokens of s[t][h],
//    p_t = e^(s[t][h] - m), l = sum_t p_t and the partial z[h][f] = sum_t p_t xf[t][f],
//    fp32, the tile's tokens in order;
//  - per (item, head): the item's tile partials combined in tile order, each scaled
//    by e^(m_tile - m_item), z_h = sum / L, then pooled_h = z_h W_v[:, 64 h .. 64 h + 63].
// Both orders are fixed, so a row never depends on the rest of the batch; an item
// with no tokens has no tiles and pools to zero.

constexpr int kPoolTile = kTileTokens;

template <int HMAX>
__global__ __launch_bounds__(256) void k_pool_part(const uint16_t *__restrict__ xf, const float *__restrict__ s,
                                                   const int *__restrict__ cu, const int2 *__restrict__ tiles, int D,
                                                   int H, float *__restrict__ zp, float2 *__restrict__ zs) {
    // LDS: weights p [256][HMAX] | z [HMAX][D] | per-wave reductions [4][HMAX]
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float *pw = lds, *zl = pw + kPoolTile * HMAX, *red = zl + HMAX * D;
    const int2 tl = tiles[blockIdx.x];
    const int c0 = tl.y, n = min(cu[tl.x + 1] - c0, kPoolTile);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // softmax statistics of the tile: thread tid holds token tid's scores
    float sv[HMAX];
#pragma unroll
    for (int h = 0; h < HMAX; ++h) sv[h] = (tid < n && h < H) ? s[(size_t)(c0 + tid) * H + h] : -INFINITY;
#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
        const float v = wave_max(sv[h]);
        if (lane == 0) red[wave * HMAX + h] = v;
    }
    __syncthreads();
    float m[HMAX];
#pragma unroll
    for (int h = 0; h < HMAX; ++h)
        m[h] = fmaxf(fmaxf(red[h], red[HMAX + h]), fmaxf(red[2 * HMAX + h], red[3 * HMAX + h]));
    __syncthreads();  // every thread has read the maxima before the sums reuse `red`
#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
        const float p = (tid < n && h < H) ? __expf(sv[h] - m[h]) : 0.f;
        pw[tid * HMAX + h] = p;
        const float v = wave_sum(p);
        if (lane == 0) red[wave * HMAX + h] = v;
    }
    __syncthreads();
    if (tid < H) {
        float mt = 0.f;
#pragma unroll
        for (int h = 0; h < HMAX; ++h)
            if (h == tid) mt = m[h];
        const float l = ((red[tid] + red[HMAX + tid]) + red[2 * HMAX + tid]) + red[3 * HMAX + tid];
        zs[(size_t)blockIdx.x * H + tid] = float2{mt, l};
    }

    // z partials: thread (slot, g) sums columns 8 g .. 8 g + 7 over tokens slot, slot + slots, ...
    const int G = D / 8, slots = kPoolTile / G;
    const int slot = tid / G, g = tid % G;
    const bool on = slot < slots;
    float acc[8][HMAX];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int h = 0; h < HMAX; ++h) acc[i][h] = 0.f;
    auto add = [&](int t, u32x4 v) {
        float p[HMAX];
#pragma unroll
        for (int h = 0; h < HMAX; h += 4) {
            const f32x4 q = *(const f32x4 *)&pw[t * HMAX + h];
            p[h] = q.x, p[h + 1] = q.y, p[h + 2] = q.z, p[h + 3] = q.w;
        }
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf16_to_f32(w4[q] & 0xffff), b = bf16_to_f32(w4[q] >> 16);
#pragma unroll
            for (int h = 0; h < HMAX; ++h) {
                acc[2 * q][h] += p[h] * a;
                acc[2 * q + 1][h] += p[h] * b;
            }
        }
    };
    if (on) {
        const uint16_t *col = xf + (size_t)c0 * D + 8 * g;
        int t = slot;
        for (; t + 3 * slots < n; t += 4 * slots) {
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = *(const u32x4 *)(col + (size_t)(t + k * slots) * D);
#pragma unroll
            for (int k = 0; k < 4; ++k) add(t + k * slots, v[k]);
        }
        for (; t < n; t += slots) add(t, *(const u32x4 *)(col + (size_t)t * D));
    }
    // the slots' partials added in slot order, then stored as whole rows
    for (int sl = 0; sl < slots; ++sl) {
        if (on && slot == sl) {
#pragma unroll
            for (int h = 0; h < HMAX; ++h)
                if (h < H) {
                    float *zr = zl + h * D + 8 * g;
#pragma unroll
                    for (int i = 0; i < 8; ++i) zr[i] = sl == 0 ? acc[i][h] : zr[i] + acc[i][h];
                }
        }
        __syncthreads();
    }
    float *zo = zp + (size_t)blockIdx.x * H * D;
    for (int i = 4 * tid; i < H * D; i += 4 * 256) *(f32x4 *)(zo + i) = *(const f32x4 *)(zl + i);
}

constexpr int kPoolMaxTiles = 128;  // tiles of one item at the largest context (32767 tokens)

__global__ __launch_bounds__(256) void k_pool_finish(const float *__restrict__ zp, const float2 *__restrict__ zs,
                                                     const int *__restrict__ itile, const uint16_t *__restrict__ wv,
                                                     void *__restrict__ out, int out_bf16, size_t out_stride, int D,
                                                     int H) {
    __shared__ float zh[1024];
    __shared__ float wt[kPoolMaxTiles];
    __shared__ float red[4][64];
    const int item = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k0 = itile[item], nk = itile[item + 1] - k0;
    char *orow = (char *)out + (size_t)item * out_stride;
    const int col = 64 * h + lane;
    if (nk == 0) {
        if (tid < 64) {
            if (out_bf16) ((uint16_t *)orow)[col] = 0;
            else ((float *)orow)[col] = 0.f;
        }
        return;
    }
    // tile weights e^(m_tile - m_item) / L, L = sum over tiles of e^(m_tile - m_item) l_tile (tile order)
    float mi = -INFINITY;
    for (int k = 0; k < nk; ++k) mi = fmaxf(mi, zs[(size_t)(k0 + k) * H + h].x);
    float L = 0.f;
    for (int k = 0; k < nk; ++k) {
        const float2 st = zs[(size_t)(k0 + k) * H + h];
        L += __expf(st.x - mi) * st.y;
    }
    const float inv = 1.0f / L;
    for (int k = tid; k < nk; k += 256) wt[k] = __expf(zs[(size_t)(k0 + k) * H + h].x - mi) * inv;
    __syncthreads();
    for (int f = tid; f < D; f += 256) {
        float z = 0.f;
        for (int k = 0; k < nk; ++k) z += wt[k] * zp[((size_t)(k0 + k) * H + h) * D + f];
        zh[f] = z;
    }
    __syncthreads();
    // pooled_h: lane = output column of the head, the four waves take quarters of the D inputs
    const int q = D / 4, f0 = wave * q;
    float acc8[8] = {};
    for (int f = f0; f < f0 + q; f += 8)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc8[k] += zh[f + k] * bf16_to_f32(wv[(size_t)(f + k) * D + col]);
    red[wave][lane] = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
    __syncthreads();
    if (wave == 0) {
        const float v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        if (out_bf16) ((uint16_t *)orow)[col] = (uint16_t)f32_to_bf16(v);
        else ((float *)orow)[col] = v;
    }
}

size_t pool_partial_bytes(int ntiles, int D, int H) { return (size_t)ntiles * H * D * 4; }
size_t pool_stats_bytes(int ntiles, int H) { return (size_t)ntiles * H * 8; }

hipError_t launch_pool(const uint16_t *xf, const float *s, const int *cu, const int2 *tiles, int ntiles,
                       const int *itile, int count, const uint16_t *wv, void *out, int out_bf16, size_t out_stride,
                       int D, int H, float *zp, float2 *zs, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    if (D % 128 || D > 1024 || H * 64 != D || H > 16) return hipErrorInvalidValue;
    if (ntiles > 0) {
        auto go = [&](auto kernel, int hmax) -> hipError_t {
            const size_t lds = ((size_t)kPoolTile * hmax + (size_t)hmax * D + 4 * (size_t)hmax) * sizeof(float);
            hipError_t e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            kernel<<<ntiles, 256, lds, stream>>>(xf, s, cu, tiles, D, H, zp, zs);
            return hipGetLastError();
        };
        hipError_t e = H <= 4 ? go(k_pool_part<4>, 4) : H <= 8 ? go(k_pool_part<8>, 8) : go(k_pool_part<16>, 16);
        if (e != hipSuccess) return e;
    }
    k_pool_finish<<<dim3(count, H), 256, 0, stream>>>(zp, zs, itile, wv, out, out_bf16, out_stride, D, H);
    return hipGetLastError();
}

}  // namespace ube
