// contrastive.h -- launch interface of the gfx950 kernels of the Matryoshka sigmoid contrastive loss
// (internal to libube).
//
// Notation: n items (pooled bf16 embeddings of D columns), R anchors = items [r0, r0 + R), K Matryoshka
// widths m_0 < ... < m_{K-1} (multiples of 64 here). Block k of the columns is [m_{k-1}, m_k) (m_{-1} = 0).
// For width w: inv_w(i) = 1 / |e_i[:m_w]| (0 for a zero prefix), s = <e_p, e_j>_w inv_w(p) inv_w(j),
// z = t s + b, sigma = 1 / (1 + exp(-z)). Dense cells are ambient negatives of weight wa; named edges,
// the item itself and padding are handled apart. c = 1 / (K R).
//   gamma = d loss / d z;  Q_w = t gamma inv_w(p) inv_w(j);  H_k = sum over w >= k of Q_w.
//   rho_w(p) = t inv_w(p)^2 sum_j gamma s;  kappa_w(j) = t inv_w(j)^2 sum_p gamma s.
//   d loss / d e_p[d in block k] = sum_j H_k(p, j) e_j[d] - (sum over w >= k of rho_w(p)) e_p[d]
//   d loss / d e_j[d in block k] = sum_p H_k(p, j) e_p[d] - (sum over w >= k of kappa_w(j)) e_j[d]
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ube {

constexpr int kMaxWidths = 8;

// One named edge after resolution: anchor p (0-based within the anchors), item j, label y (+1 attract,
// -1 repel, 0 ignore) and weight w.
struct ContrastiveEdge {
    int p, j, y;
    float w;
};

struct ContrastiveArgs {
    const uint16_t *emb;  // [n x ld] bf16 rows
    size_t ld;            // elements
    int n, R, r0, D, K;
    int n_pad, R_pad;     // multiples of 256
    int widths[kMaxWidths];
    float t, b, wa, c;
    bool dense;           // ambient cells present (ambient negatives with a non-zero weight)
    float *inv;           // [K][n]
    uint16_t *H;          // [K][R_pad][n_pad]
    float *rowpart;       // [n_pad / 128][K][R_pad]: sum over a 128-item tile of gamma s
    float *colpart;       // [R_pad / 128][K][n_pad]: sum over a 128-anchor tile of gamma s
    float *wgpart;        // [tiles][K][2]: c wa sum sigma, wa ln2 sum log2(1 + 2^z2)
    // named edges
    const ContrastiveEdge *edges;
    int E;
    const uint32_t *row_edges;   // [R + 1] offsets of each anchor's edges (edges sorted by anchor)
    const uint32_t *col_offsets; // [n + 1] offsets into col_edges
    const uint32_t *col_edges;   // [E] edge indices grouped by item, ascending anchor within an item
    float *edge_out;             // [E][4][K]: delta gamma s, delta gamma, delta loss, delta H (per block)
    // reductions
    float *rho;        // [K][R_pad]: rho of each width
    float *rsum;       // [K][R_pad]: sum over the anchor's row of gamma s, per width
    float *kappa_blk;  // [K][n_pad]: block coefficients of kappa (sums over widths w >= k)
    float *scalars;    // [3 + K]: loss, d/dt, d/db, width losses
    bool want_loss;
    // gradient
    int splits, chunk;     // split of the items for the rows contraction
    float *rows_partial;   // [splits][R_pad][D]
    float *rows_final;     // [R_pad][D]
    float *grad;           // [n x gld] fp32
    size_t gld;            // elements
    const uint32_t *touched;  // items with named edges (as anchor or as candidate)
    int T;
};

hipError_t launch_prefix_inv_norms(const ContrastiveArgs &a, hipStream_t stream);
hipError_t launch_contrastive_edges(const ContrastiveArgs &a, hipStream_t stream);
hipError_t launch_contrastive_cells(const ContrastiveArgs &a, bool grad, hipStream_t stream);
hipError_t launch_contrastive_reduce(const ContrastiveArgs &a, bool grad, hipStream_t stream);
// rows contraction (split over items) and its finish: rows_final = sum of splits - rho terms
hipError_t launch_contrastive_grad_rows(const ContrastiveArgs &a, hipStream_t stream);
// columns contraction writing the gradient (or, without dense cells, the rho / kappa terms alone)
hipError_t launch_contrastive_grad_cols(const ContrastiveArgs &a, hipStream_t stream);
// named-edge terms added onto the gradient rows of the touched items
hipError_t launch_contrastive_sparse(const ContrastiveArgs &a, hipStream_t stream);
// no anchors: zero loss and gradient
hipError_t launch_contrastive_empty(const ContrastiveArgs &a, hipStream_t stream);

}  // namespace ube
