// Internal declarations shared by the library's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pma.h"

namespace pma {

// ---- index build (index_build.hip) ---------------------------------------

// Zero entries kept after the last source index (see GraphDev::csr_src).
constexpr int kSrcPad = 16;
// rows the q-projecting edge kernel keeps in LDS (64 x 2 KB per workgroup)
constexpr int kHotRows = 64;
// The backward's source pieces are grouped into kBands bands of targets with
// equal edge counts, one band per XCD (an MI355X has 8).
constexpr int kBands = 8;

// Device arrays describing one graph; owned by the plan.
struct GraphDev {
    int32_t *row_ptr = nullptr;   // L + 1
    int32_t *csr_src = nullptr;   // nnz (+ kSrcPad zeros), per target ascending source
    int32_t *csr_tgt = nullptr;   // nnz
    int32_t *csr_eid = nullptr;   // nnz (+ kSrcPad zeros), position in the edge order
    int32_t *task_target = nullptr, *task_begin = nullptr, *task_end = nullptr,
            *task_slot = nullptr, *task_split = nullptr; // n_tasks each; split index or -1
    int32_t *split_target = nullptr, *split_slot0 = nullptr, *split_count = nullptr; // n_split
    // Sources some edge reads, in ascending order (kv_rows[0, n_kv)), and each
    // CSR entry's source as a position in that list (csr_kv, + kSrcPad zeros).
    int32_t *kv_rows = nullptr, *csr_kv = nullptr;
    // Source-major view, built on first use by a backward pass: per source s
    // its entries csc_ptr[s] .. csc_ptr[s+1] give each edge's target
    // (csc_tgt), its position in the target-grouped arrays (csc_pos) and in
    // the edge order (csc_eid). csc_tgt, csc_pos and csc_eid carry kSrcPad
    // zero entries past nnz.
    int32_t *csc_ptr = nullptr, *csc_tgt = nullptr, *csc_pos = nullptr, *csc_eid = nullptr;
    // Source pieces, built with the source-major view: piece i covers entries
    // s_begin[i] .. s_end[i] of source s_source[i]; s_slot[i] is its partial
    // slot, -1 when the source is one piece. Sources in more than one piece:
    // ss_source, with slots ss_slot0 .. ss_slot0 + ss_count - 1. A piece lies
    // within one band of targets; pieces are ordered by band, then by their
    // first target; band k holds pieces s_band_off[k] .. s_band_off[k+1].
    int32_t *s_source = nullptr, *s_begin = nullptr, *s_end = nullptr, *s_slot = nullptr;
    int32_t *ss_source = nullptr, *ss_slot0 = nullptr, *ss_count = nullptr;
    int64_t n_tasks = 0, n_split = 0, n_slots = 0, max_degree = 0, n_kv = 0;
    int64_t n_stasks = 0, n_ssplit = 0, n_sslots = 0;
    int64_t s_band_off[kBands + 1] = {0};
    bool s_banded = false;        // false: one band (no source long enough to cut)
};

// Builds every array of GraphDev from host edges (already validated, loops
// appended). Returns PMA_OK, PMA_E_INDEX_DUPLICATE, PMA_E_OOM or
// PMA_E_DEVICE. Blocks on `stream` once. On failure frees what it made.
pma_status build_graph(const int32_t *h_src, const int32_t *h_tgt, int64_t nnz, int64_t L,
                       int64_t S, int chunk, hipStream_t stream, GraphDev *g, char *err,
                       size_t errlen);
void free_graph(GraphDev *g);
// Builds the source-major view and the source pieces of at most `chunk`
// entries, banded (blocks on `stream`).
pma_status build_csc(GraphDev *g, int64_t nnz, int64_t L, int64_t S, int chunk, int sub,
                     hipStream_t stream, char *err, size_t errlen);

// ---- projections (proj.hip) ----------------------------------------------

// Output block of a projection launch: y = x W^T + b written at
// dst + b_idx * sb + i_idx * si (elements), row of E channels.
struct ProjOut {
    const void *w;   // (E, E) [out][in]
    const void *b;   // (E) or nullptr
    void *dst;
    int64_t sb, si;  // element strides of the sample and token index
};

// Rows are visited in iteration order r = 0 .. rows-1, where r stands for
// (sample b, token i) as
//   token_major == 0:  r = b * n + i
//   token_major == 1:  r = i * B + b
// and the input row of (b, i) is x + (b * n + i) * E when x_token_major == 0
// (batch-first tokens), x + (i * B + b) * E when 1 (target-major layout).
struct ProjArgs {
    const void *x;
    int64_t rows;     // B * n
    int64_t n, B;
    int token_major;
    int nblk;         // 1..3 output blocks
    ProjOut out[3];
    int x_token_major = -1;  // -1: same as token_major (rows read in storage order)
    // With a row list, iteration token i of sample b reads input row
    // b * n_in + row_list[i] (batch-first input of n_in tokens per sample).
    const int32_t *row_list = nullptr;
    int64_t n_in = 0;
    int x3 = 0;       // fp32, embed_dim 128: split-bf16 matrix-core products (proj_x3)
};

pma_status launch_proj(const ProjArgs &a, int64_t E, pma_dtype dt, hipStream_t s);

// ---- edge attention (edge.hip) -------------------------------------------

// Element strides of the workspace tensors. Target-major: q and mixed
// [L][B][E], keys and values [S][2][B][E] (one source's keys for all samples,
// then its values). Batch-first: q and mixed [B][L][E], keys [B][S][E]
// followed by values [B][S][E].
struct Layout {
    int64_t q_t, q_b;           // q row of (target t, sample b) at t*q_t + b*q_b
    int64_t kv_s, kv_b, kv_v;   // key row of (source s, sample b) at s*kv_s + b*kv_b; values +kv_v
    int64_t m_t, m_b;           // mixed row of (t, b) at t*m_t + b*m_b
};
Layout make_layout(bool batch_first, int64_t B, int64_t L, int64_t S, int64_t E);

struct EdgeArgs {
    const GraphDev *g;
    const int32_t *gather_src;  // per CSR entry, the key/value workspace row it reads
    int64_t B, L, S, E, H, nnz;
    pma_dtype dt;
    Layout lay;
    const void *qt;     // q rows (layout lay)
    const void *kv;     // key and value rows (layout lay)
    uint64_t kv_bytes = 0;  // size of kv
    void *mixed;        // mixed rows (layout lay)
    float *part_acc;    // [slot][B][E]
    float *part_ml;     // [slot][B][H][2]
    float *stat_ml;     // [L][B][H][2] final (max, sum) or nullptr
    float *scores;      // [nnz][B][H] log2-domain scores by CSR position, or nullptr
    float *weights;     // caller's weights or nullptr
    int average;
    int xcd_map = 1;    // 1: sample group fixed per XCD where the group count
                        // divides 8; 2: groups in turn; 0: interleaved
    int nt = 0;         // bit 0: non-temporal q loads, bit 1: non-temporal mixed / out stores
    const uint64_t *kpm_bits = nullptr;  // key_padding_mask bits (pack_mask layout)
    const uint32_t *kpm_csr = nullptr;   // the same by CSR position (gather_mask)
    int kpm_w32 = 0;                     // its 32-bit words per position
    int kpm_words = 0;                   // 64-bit words per source
    int persist = 0;    // edge kernel: workgroups per CU, each wavefront walking
                        // several pieces (0: one wavefront per piece and pass)
    // out_proj fused into the edge and merge kernels (out_fusable)
    int fuse_out = 0;
    const void *wo = nullptr, *bo = nullptr;
    // q = query Wq^T + bq inside the edge kernel (needs fuse_out); qt and
    // lay then address the caller's (B, L, E) query tokens
    int fuse_in = 0;
    const void *wq = nullptr, *bq = nullptr;
    void *out = nullptr;
    // hot-row cache of the q-projecting edge kernel: gather_src with ~slot for
    // the edges of the n_hot rows hot_src[slot] (nullptr: no cache)
    const int32_t *hot_csr = nullptr, *hot_src = nullptr;
    int n_hot = 0;
    // split targets merged inside the edge kernel where each has at most 4
    // pieces (max_pieces: the most pieces of one target; see edge_fast)
    int coop = 0;
    int max_pieces = 0;
};

// Whether edge_fast / merge_fast can apply out_proj themselves.
bool out_fusable(int64_t E, int64_t H, pma_dtype dt);
// Whether edge_fast can also project q itself (with out_proj fused).
bool q_fusable(int64_t E, int64_t H, pma_dtype dt);

// key_padding_mask bytes (sample b's S bytes at mask + b * bstride; bstride
// 0 for one shared mask) -> bits[s * words + b / 64], bit b % 64, words =
// ceil(B / 64). Asynchronous on s.
pma_status pack_mask(const uint8_t *mask, int64_t bstride, int64_t B, int64_t S, uint64_t *bits,
                     hipStream_t s);
// bits by CSR position in 32-bit words (w32 = ceil(B / 32) per position):
// out[p * w32 + j] = half j % 2 of bits[src[p] * words + j / 2].
pma_status gather_mask(const uint64_t *bits, int words, int w32, const int32_t *src, int64_t nnz,
                       uint32_t *out, hipStream_t s);

// ---- backward pass (backward.hip) ------------------------------------------

struct BwdArgs {
    int B, L, S, E, H;
    float scale_log2;    // log2(e) / sqrt(d): the forward's score scale
    float inv_sqrt_d;
    const void *q, *k, *v, *mixed;   // saved, batch-first, plan dtype
    // non-temporal: target-pass loads of mixed (bit 0), of q and dm (bit 1),
    // source-pass key / value loads (bit 2), dq / dk / dv stores (bit 3)
    int nt = 0;
    int Skv;                         // key/value rows per sample in the save area
    const int32_t *kv_src;           // per CSR entry, its key/value row there
    const float *ml;                 // saved [L][B][H][2] (max, sum), base 2
    const void *dm;                  // (B, L, E) gradient reaching mixed, plan dtype
    const int32_t *row_ptr, *csr_src, *csc_ptr, *csc_tgt, *csc_pos;
    // target pieces (the forward's) and source pieces, with their splits
    const int32_t *t_target, *t_begin, *t_end, *t_slot;
    const int32_t *ts_target, *ts_slot0, *ts_count;
    const int32_t *s_source, *s_begin, *s_end, *s_slot;
    const int32_t *ss_source, *ss_slot0, *ss_count;
    int64_t n_ttasks, n_tsplit, n_stasks, n_ssplit;
    int64_t n_tslots, n_sslots;      // partial slots of the split targets / sources
    int64_t s_band_off[kBands + 1];  // source pieces per band (one band per XCD)
    int banded;                      // 0: one band, launched in plain order
    // banded source pass: 2 = sample groups in turn within each band (the
    // band's wavefronts for group 0, then group 1, ...), 0 = interleaved
    int s_order = 2;
    // target pass order over sample groups of 64 lanes (t_groups of them):
    // 0 interleaved, 1 group g on the XCDs x with x % t_groups = g (t_groups
    // divides 8), 2 groups in turn, -1 chosen at launch; t_gthreads threads
    // per group (whole workgroups)
    int t_order, t_groups;
    int t_pf = -1;       // target pass: next rows requested ahead (1), not (0), automatic (-1)
    int64_t t_gthreads;
    const uint64_t *kpm_bits;        // packed mask or nullptr
    int kpm_words;
    const uint32_t *kpm_csr;         // the mask by CSR position (gather_mask), or nullptr
    int kpm_w32;
    void *PZ;                        // per-channel path: [nnz][B][H] (p, dz) pairs, bf16 for bf16 plans
    float *mD;                       // 16-byte path: [L][B][H] (m + log2 l, D) from the target pass
    float *part_q;                   // [target slot][B][E] partial dq
    float *part_kv;                  // [source slot][B][2E] partial dk, dv
    void *dq, *dk, *dv;              // (B, L, E), (B, S, E), (B, S, E), plan dtype
};
// Whether the backward's edge passes take the 16-byte kernels (which need no
// per-edge (p, dz) array) for these sizes and saved tensors.
bool bwd_edges_fast(int64_t E, int64_t H, pma_dtype dt, const void *q, const void *k,
                    const void *v, const void *mixed);
pma_status launch_bwd_edges(const BwdArgs &a, pma_dtype dt, hipStream_t s);
// fp32 bytes of part_q + part_kv
size_t bwd_piece_scratch(const GraphDev &g, int64_t B, int64_t E);

// y (rows, E) = sum_j x_j (rows, E) W_j with W_j (E, E) [out][in]: the
// gradient of x W^T with respect to x, summed over the maps that read x.
// accumulate: y += (fp32 plans only). Row-major, plan dtype.
struct RowMM {
    const void *x[3];
    const void *w[3];
    int nin;
    void *y;
    int64_t rows;
    int accumulate;
};
pma_status launch_rowmm(const RowMM &a, int64_t E, pma_dtype dt, hipStream_t s);

// Weight and bias gradients of up to four linear maps y = x W^T + b:
// dW = G^T X (E, E) [out][in] and db = column sums of G (skipped when db is
// null), with G = dy and X = x (rows, E) row-major; plan dtype in and out.
struct WGradPair {
    const void *g, *x;
    int64_t rows;
    void *dw, *db;
    // With a row list (B * n_in < 2^31), pair row r = b * n + i reads row
    // b * n_in + list[i] of G and of X: the rows of the other tokens are zero
    // in G (sources that no edge reads) and are skipped.
    const int32_t *list = nullptr;
    int64_t n = 0, n_in = 0;
};
struct WGrad {
    WGradPair p[4];
    int np;
    int E;
    int nwg;        // set by launch_wgrad: workgroups over all pairs,
    int nwg_p[4];   // of pair i (in proportion to its rows),
    int off_p[4];   // the first of pair i
    float *part;    // wgrad_scratch bytes
};
size_t wgrad_scratch(int64_t E, int np, int64_t max_rows);
pma_status launch_wgrad(WGrad a, pma_dtype dt, hipStream_t s);

// ---- PackedLinear (linear.hip) ----------------------------------------------
// A node's row is R values in segments of Cs: value (segment b, k) of node n
// sits at n * sn + b * sb + k (node-major rows: Cs = R, sn = R; batch-first
// tensors: Cs = C, sn = C, sb = nodes * C). y rows = sum over the entries of
// each output row's pieces of w[eid] x rows[idx] (+ bias[row] on every
// value); plan dtype in and out.
struct LinArgs {
    int R, Cs;
    int64_t sn_in, sb_in, sn_out, sb_out;
    const void *x, *w, *bias;      // bias (rows_out) or nullptr
    void *y;
    const int32_t *idx, *eid;      // per entry: input row, position in the edge order
    const int32_t *t_row, *t_begin, *t_end, *t_slot;
    int64_t n_tasks;
    const int32_t *s_row, *s_slot0, *s_count;
    int64_t n_split;
    float *part;                   // [slot][R]
    int nseg = 1, cgp = 64;        // set by the launcher
};
// dw_e = dot(dy row of t_e, x row of s_e), edge order; db[t] = sum of the dy
// row of t when db is not null.
struct RowDots {
    const int32_t *csr_src, *csr_tgt, *csr_eid;
    int64_t nnz, L;
    int R, Cs;
    int64_t snx, sbx, sng, sbg;
    const void *x, *dy;
    void *dw, *db;
    int cgp = 64;                  // set by the launcher
};
// Values per lane: 16 bytes when Cs fills whole 16-byte chunks and every
// pointer is 16-byte aligned, else 1.
int lin_vec(int64_t Cs, pma_dtype dt, const void *const *ptrs, int n);
pma_status launch_spmm(const LinArgs &a, pma_dtype dt, int vec, hipStream_t s);
pma_status launch_lin_rowdots(const RowDots &a, pma_dtype dt, int vec, hipStream_t s);
// out[q][p][c] = in[p][q][c]
pma_status launch_transpose(const void *in, void *out, int64_t P, int64_t Q, int64_t C,
                            pma_dtype dt, hipStream_t s);

// Whether the edge kernels take a key_padding_mask for these arguments (the
// fast kernel needs every tensor under 2 GiB when masked).
bool mask_supported(const EdgeArgs &x);
pma_status launch_edge(const EdgeArgs &a, hipStream_t s);

pma_status launch_merge(const EdgeArgs &a, hipStream_t s);
// The edge kernel's loads alone (calibration; see gather_probe in edge.hip).
// PMA_E_UNSUPPORTED where the 16-byte kernel does not serve the head size or
// a tensor is 2 GiB or more.
pma_status launch_gather_probe(const EdgeArgs &a, hipStream_t s);
// Whether launch_edge merges the split targets itself (then no launch_merge).
bool edge_merges_splits(const EdgeArgs &a);
// Calibration: n 1 KB row gathers from a table (pma_gather_ceiling).
pma_status launch_gather_ceiling(const void *table, uint64_t table_bytes, const int32_t *rows,
                                 int64_t n, int64_t per, void *sink, hipStream_t s);
pma_status launch_weights(const EdgeArgs &a, hipStream_t s);

}  // namespace pma
