/*
 * pma.h -- packed multi-head attention over live edges, for AMD MI355X (gfx950).
 *
 * Each target token attends only to its listed sources. For every live edge
 * e from source s to target t, each head scores dot(q[t], k[s]) / sqrt(d);
 * a softmax over the edges into each target turns the scores into weights;
 * the weights mix the sources' values; the heads are joined and passed
 * through out_proj. q, k, v and out come from four embed_dim x embed_dim
 * projections shared by every node and edge. (kpnn2 0.3.0 API reference,
 * PackedMultiheadAttention: class docstring and "Notes", steps 1-5.)
 * Dense nn.MultiheadAttention is the special case of a complete graph
 * (continuiti MultiHeadAttention page: MultiHead = Concat(head_i) W^O + b^O).
 *
 * Conventions shared by every call:
 *   - L = query_features (tokens that attend), S = key_features (tokens
 *     attended to), E = embed_dim, H = num_heads, d = E / H. Head h uses
 *     channels [h d, (h + 1) d) of each projection.
 *   - A projection is y = x W^T + b with W stored row-major [out][in]
 *     (E x E) and b of length E, as nn.Linear stores it.
 *   - Tokens are batch-first and contiguous: query (B, L, E), key and value
 *     (B, S, E), out (B, L, E), where B is the product of the leading axes
 *     (1 for unbatched input). The graph is shared by all B samples.
 *   - Floating-point tensors (tokens, weights, biases, out) all have the
 *     plan's dtype. Products and sums accumulate in fp32; with PMA_BF16 the
 *     library keeps its q, k, v and mixed intermediates in bf16 (round to
 *     nearest even) and rounds out the same way.
 *   - Every call returns a status and never throws. On failure,
 *     pma_last_error() holds a message for the calling thread.
 */
#ifndef PMA_H
#define PMA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pma_plan pma_plan; /* opaque */

typedef enum {
    PMA_F32 = 0,  /* fp32 tokens and parameters */
    PMA_BF16 = 1  /* bf16 tokens and parameters, fp32 softmax and accumulation */
} pma_dtype;

typedef enum {
    PMA_OK = 0,
    PMA_E_NULL = 1,            /* a required pointer is NULL */
    PMA_E_SIZE = 2,            /* a size is not positive, or E % H != 0 */
    PMA_E_INDEX_EMPTY = 3,     /* nnz < 1 */
    PMA_E_INDEX_RANGE = 4,     /* a source >= S or a target >= L, or negative */
    PMA_E_INDEX_DUPLICATE = 5, /* a (source, target) pair occurs twice */
    PMA_E_SELF_LOOPS = 6,      /* add_self_loops with L != S */
    PMA_E_DTYPE = 7,           /* not a pma_dtype value */
    PMA_E_ARG = 8,             /* another invalid argument (flag, bias pointers) */
    PMA_E_OOM = 9,             /* a host or device allocation failed */
    PMA_E_DEVICE = 10,         /* a HIP call or kernel launch failed */
    PMA_E_UNSUPPORTED = 11     /* sizes beyond the library's 32-bit edge indexing */
} pma_status;

/* Stages that pma_profile_read reports, in launch order. */
typedef enum {
    PMA_STAGE_PROJ_IN = 0, /* q, k and v projections */
    PMA_STAGE_EDGE = 1,    /* score, online softmax and mix over the edges; when
                              out_proj is fused (embed_dim 64) also out_proj */
    PMA_STAGE_MERGE = 2,   /* merge of targets split into several pieces; when
                              out_proj is fused also their out_proj */
    PMA_STAGE_WEIGHTS = 3, /* need_weights: one weight per live edge */
    PMA_STAGE_OUT = 4,     /* out_proj when it is not fused */
    PMA_NUM_STAGES = 5
} pma_stage;

/*
 * pma_create -- build a plan for one graph.
 *
 * Follows the kpnn2 PackedMultiheadAttention constructor (parameter table and
 * "Raises"): source_index[i] is the key/value position that edge i reads from
 * (0 <= source < key_features), target_index[i] the query position that
 * attends along it (0 <= target < query_features); the two arrays pair up by
 * position, hold nnz >= 1 entries and must not repeat a (source, target) pair.
 * embed_dim must be divisible by num_heads. With add_self_loops != 0 (which
 * needs query_features == key_features) every missing pair (i, i) is appended
 * after the given pairs, in ascending i; existing loops are kept, not
 * duplicated. The edge order so formed is the order of the per-edge weights
 * pma_forward returns.
 *
 *   plan            out: the new plan, or NULL on failure.
 *   source_index,   HOST arrays of nnz int64; read during the call and
 *   target_index    copied, never modified or retained.
 *   nnz             number of given pairs.
 *   query_features  L; key_features S; embed_dim E; num_heads H (all > 0).
 *   add_self_loops  0 or 1.
 *   dtype           dtype of every floating-point tensor used with the plan.
 *   stream          stream for the device-side index build. The call blocks
 *                   until that build finishes (it reads back a duplicate flag).
 *
 * Errors: PMA_E_NULL, PMA_E_SIZE, PMA_E_INDEX_EMPTY, PMA_E_INDEX_RANGE,
 * PMA_E_INDEX_DUPLICATE, PMA_E_SELF_LOOPS, PMA_E_DTYPE, PMA_E_ARG (flag not
 * 0/1), PMA_E_UNSUPPORTED (nnz, L or S beyond 2^31 - 1 entries), PMA_E_OOM,
 * PMA_E_DEVICE. On any error nothing stays allocated and *plan is NULL.
 * Argument errors are detected before any HIP call.
 */
pma_status pma_create(pma_plan **plan, const int64_t *source_index, const int64_t *target_index,
                      int64_t nnz, int64_t query_features, int64_t key_features,
                      int64_t embed_dim, int64_t num_heads, int add_self_loops, pma_dtype dtype,
                      hipStream_t stream);

/*
 * pma_forward -- one forward pass over a batch (kpnn2 page, forward, and
 * "Notes" steps 1-5).
 *
 *   batch           B > 0: samples in the leading axes (1 if unbatched).
 *   query           DEVICE (B, L, E); key, value DEVICE (B, S, E). They may
 *                   be the same pointer (attention within one graph); the
 *                   library then projects each token row once.
 *   q_w, k_w, v_w,  DEVICE (E, E) [out][in] projection weights.
 *   o_w
 *   q_b, k_b, v_b,  DEVICE (E) biases: all four given, or all four NULL
 *   o_b             (bias = False).
 *   out             DEVICE (B, L, E). A target with no live edge gets exactly
 *                   o_b (zeros without bias): it mixes to zeros, not NaN.
 *   weights         NULL (need_weights = False), or DEVICE fp32 receiving the
 *                   softmax weight of every live edge in edge order: (B, nnz)
 *                   averaged over heads when average_attn_weights != 0, else
 *                   (B, nnz, H). Weights into one target sum to 1.
 *   stream          all work is enqueued on this stream; the call does not
 *                   synchronise (except the first time a larger batch needs
 *                   a larger workspace, which waits for the stream before
 *                   reallocating).
 *
 * Tokens, parameters, out and weights are borrowed: they belong to the
 * caller and must stay valid until the enqueued work completes. A plan must
 * not run two forwards at once (they share the plan's workspace). Inputs
 * must not overlap out or weights.
 *
 * Errors: PMA_E_NULL (plan, a token, a weight or out is NULL), PMA_E_SIZE
 * (batch <= 0), PMA_E_ARG (biases neither all given nor all NULL, flag not
 * 0/1), PMA_E_OOM, PMA_E_DEVICE.
 */
pma_status pma_forward(pma_plan *plan, int64_t batch, const void *query, const void *key,
                       const void *value, const void *q_w, const void *q_b, const void *k_w,
                       const void *k_b, const void *v_w, const void *v_b, const void *o_w,
                       const void *o_b, void *out, float *weights, int average_attn_weights,
                       hipStream_t stream);

/*
 * pma_forward_static -- pma_forward that allocates nothing, for callers that
 * cannot allocate device memory during the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and errors as pma_forward, plus PMA_E_SIZE (below).
 *
 * Its workspace (the projected keys and values; q and the mixed rows where
 * they are not fused away; the partial results of split targets; with
 * weights the scores and softmax statistics) is carved from one file-scope
 * device array of PMA_STATIC_SCRATCH_BYTES, which each GPU the library runs
 * on holds from the library's first use on it until the process ends. The
 * plan's own workspace is neither used nor grown, and no stage timing is
 * recorded. A forward that would need more than the array fails with
 * PMA_E_SIZE before any launch (the 20,000-node gene workload at batch 32,
 * embed_dim 64, bf16 needs about 67 MB; the bipartite and 100k-node
 * workloads need more and are refused).
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (on other streams, from other
 * threads, with other plans) race with each other, so the caller must order
 * them (e.g. one stream).
 */
#define PMA_STATIC_SCRATCH_BYTES ((size_t)96 << 20)

pma_status pma_forward_static(pma_plan *plan, int64_t batch, const void *query, const void *key,
                              const void *value, const void *q_w, const void *q_b,
                              const void *k_w, const void *k_b, const void *v_w, const void *v_b,
                              const void *o_w, const void *o_b, void *out, float *weights,
                              int average_attn_weights, hipStream_t stream);

/*
 * pma_forward_masked -- pma_forward with a key_padding_mask (kpnn2 page,
 * forward parameter table, key_padding_mask; "Notes" step 3 and the
 * paragraph on queries with no live keys).
 *
 *   key_padding_mask  DEVICE bytes, one per key (source token): (B, S) when
 *                     mask_per_sample = 1, else (S,) shared by every sample.
 *                     Nonzero leaves that key out of the sample: the edges
 *                     from it drop out of the softmax (weight 0) and the
 *                     other edges into the same target share the whole
 *                     weight. A target whose keys are all masked mixes to
 *                     zeros, so its output is o_b. Borrowed like the tokens.
 *   mask_per_sample   0 or 1.
 *   other arguments   as pma_forward.
 *
 * Errors: those of pma_forward, and PMA_E_NULL (key_padding_mask NULL),
 * PMA_E_ARG (mask_per_sample not 0/1), PMA_E_UNSUPPORTED (a workspace tensor
 * of 2 GiB or more with a head size the 16-byte kernel serves, or
 * nnz * ceil(batch / 32) of 2^31 or more).
 */
pma_status pma_forward_masked(pma_plan *plan, int64_t batch, const void *query, const void *key,
                              const void *value, const void *q_w, const void *q_b,
                              const void *k_w, const void *k_b, const void *v_w, const void *v_b,
                              const void *o_w, const void *o_b, void *out, float *weights,
                              int average_attn_weights, const uint8_t *key_padding_mask,
                              int mask_per_sample, hipStream_t stream);

/* ---- training ------------------------------------------------------------
 *
 * The kpnn2 page's layer trains through torch autograd ("Notes": training
 * keeps the gathers, or recomputes them, for backward). Here a forward that
 * will be differentiated writes what the backward needs to a caller-owned
 * save area, and pma_backward returns the gradients of every input and
 * parameter. Dropout is not applied (eval-mode softmax).
 */

/* Bytes of the save area for a batch of `batch` samples (0 for a NULL plan
   or batch <= 0). */
size_t pma_train_bytes(const pma_plan *plan, int64_t batch);

/*
 * pma_forward_train -- pma_forward (masked when key_padding_mask is not
 * NULL) that also fills `save` (DEVICE, pma_train_bytes(plan, batch) bytes,
 * 256-byte aligned): the projected q, k, v, the joined mix before out_proj
 * and each target's softmax statistics. The save area belongs to the caller
 * and must stay unchanged until the matching pma_backward. Errors: those of
 * pma_forward_masked, and PMA_E_NULL (save NULL).
 */
pma_status pma_forward_train(pma_plan *plan, int64_t batch, const void *query, const void *key,
                             const void *value, const void *q_w, const void *q_b, const void *k_w,
                             const void *k_b, const void *v_w, const void *v_b, const void *o_w,
                             const void *o_b, void *out, float *weights, int average_attn_weights,
                             const uint8_t *key_padding_mask, int mask_per_sample, void *save,
                             hipStream_t stream);

/*
 * pma_backward -- gradients of sum(out * grad_out) for the forward that
 * filled `save` (same plan, batch, tokens, weights and mask).
 *
 *   query, key, value, q_w, k_w, v_w, o_w   DEVICE, as given to the forward.
 *   has_bias          1 if the forward had biases (then the four bias
 *                     gradients are written), else 0.
 *   grad_out          DEVICE (B, L, E), plan dtype.
 *   key_padding_mask, mask_per_sample       as given to the forward (NULL
 *                     for none).
 *   grad_query (B, L, E), grad_key, grad_value (B, S, E), grad_*_w (E, E),
 *   grad_*_b (E)      DEVICE outputs in the plan dtype, overwritten. When
 *                     two of query / key / value are one tensor, pass one
 *                     output pointer for both: it receives the sum of their
 *                     gradients.
 *
 * Computation: out_proj gradients, then two passes over the edges (by
 * target: query gradients and each edge's softmax weight and score
 * gradient; by source: key and value gradients), then the projections'
 * gradients; fp32 accumulation throughout, intermediates in the plan dtype,
 * every product on this library's own matrix-core kernels, no atomics
 * (results are run-to-run identical). The first call builds a source-major
 * copy of the edge index (blocks once). Errors: PMA_E_NULL, PMA_E_SIZE,
 * PMA_E_ARG (flags, a shared gradient output with L != S),
 * PMA_E_UNSUPPORTED (head size above 64; a mask with nnz * ceil(batch / 32)
 * of 2^31 or more), PMA_E_OOM, PMA_E_DEVICE.
 */
pma_status pma_backward(pma_plan *plan, int64_t batch, const void *query, const void *key,
                        const void *value, const void *q_w, const void *k_w, const void *v_w,
                        const void *o_w, int has_bias, const void *save, const void *grad_out,
                        const uint8_t *key_padding_mask, int mask_per_sample, void *grad_query,
                        void *grad_key, void *grad_value, void *grad_q_w, void *grad_q_b,
                        void *grad_k_w, void *grad_k_b, void *grad_v_w, void *grad_v_b,
                        void *grad_o_w, void *grad_o_b, hipStream_t stream);

/* ---- PackedLinear on the same packed pairs ------------------------------ */

/*
 * The kpnn2 PackedMultiheadAttention page ("See also") describes PackedLinear
 * as the same packed pairs with one trained scalar per edge, the same for
 * every sample, information flowing from source to target. Read as a linear
 * map whose (L x S) weight matrix holds w_e at each live pair (t_e, s_e) and
 * zero elsewhere, applied to every sample b and channel c:
 *
 *   out[b, t, c] = bias[t] + sum over edges e into t of w_e x[b, s_e, c].
 *
 * channels = 1 is the nn.Linear-shaped layer (in_features = S nodes,
 * out_features = L nodes); more channels apply the same map to each.
 *
 * pma_create_graph -- a plan for these calls only: pma_create's index rules
 * and edge order (given pairs, then appended loops when add_self_loops), no
 * attention sizes. The attention calls reject it with PMA_E_ARG. A plan
 * from pma_create serves the PackedLinear calls as well.
 */
pma_status pma_create_graph(pma_plan **plan, const int64_t *source_index,
                            const int64_t *target_index, int64_t nnz, int64_t query_features,
                            int64_t key_features, int add_self_loops, pma_dtype dtype,
                            hipStream_t stream);

/*
 * pma_linear_forward -- out = the map above.
 *
 *   batch, channels  B > 0 and C > 0.
 *   x                DEVICE (B, S, C), plan dtype, contiguous.
 *   weight           DEVICE (nnz) plan dtype: weight[i] belongs to edge i of
 *                    the edge order (pma_edges).
 *   bias             DEVICE (L) plan dtype, or NULL (no bias).
 *   out              DEVICE (B, L, C) plan dtype. A target with no edge gets
 *                    bias[t] (zero without bias).
 *
 * Sums are fp32, in each target's ascending-source order (pieces of long
 * targets summed in order). Enqueued on `stream`; scratch for split targets
 * is grown (blocking once) when a larger B * C needs it. Errors: PMA_E_NULL,
 * PMA_E_SIZE, PMA_E_UNSUPPORTED (B * C beyond 2^31 - 1), PMA_E_OOM,
 * PMA_E_DEVICE.
 */
pma_status pma_linear_forward(pma_plan *plan, int64_t batch, int64_t channels, const void *x,
                              const void *weight, const void *bias, void *out,
                              hipStream_t stream);

/*
 * pma_linear_backward -- gradients of sum(out * grad_out) for the same call:
 *   grad_x[b, s, c]  = sum over edges e out of s of w_e grad_out[b, t_e, c]
 *                      (zero for a source no edge reads), DEVICE (B, S, C);
 *   grad_weight[i]   = sum over b, c of grad_out[b, t_i, c] x[b, s_i, c],
 *                      DEVICE (nnz), edge order;
 *   grad_bias[t]     = sum over b, c of grad_out[b, t, c], DEVICE (L), or
 *                      NULL to skip it.
 * The first call builds the plan's source-major index (blocking once).
 * Errors as pma_linear_forward.
 */
pma_status pma_linear_backward(pma_plan *plan, int64_t batch, int64_t channels, const void *x,
                               const void *weight, const void *grad_out, void *grad_x,
                               void *grad_weight, void *grad_bias, hipStream_t stream);

/* pma_destroy -- free the plan and everything it owns. NULL is a no-op.
   Waits for the device before freeing. */
pma_status pma_destroy(pma_plan *plan);

/*
 * pma_edge_list -- the edge order a plan for these indices would have,
 * computed on the host alone (no HIP call; for callers that validate and
 * store a graph before any GPU is involved). The same rules as pma_create
 * (kpnn2 page, constructor parameter table and "Raises"): nnz >= 1, sources
 * in [0, key_features), targets in [0, query_features), no repeated
 * (source, target) pair, add_self_loops (0 or 1) only with query_features
 * == key_features; the given pairs in order, then with add_self_loops every
 * missing (i, i) in ascending i.
 *
 *   source_index, target_index  HOST, nnz int64 each; read only.
 *   capacity        entries src_out and tgt_out can hold (nnz + L always
 *                   suffices).
 *   src_out, tgt_out HOST outputs: the final edge list.
 *   nnz_out         HOST: its length (also set when capacity is too small).
 *
 * Errors: PMA_E_NULL, PMA_E_SIZE (a size <= 0, or capacity below the list's
 * length), PMA_E_INDEX_EMPTY, PMA_E_INDEX_RANGE, PMA_E_INDEX_DUPLICATE,
 * PMA_E_SELF_LOOPS, PMA_E_ARG, PMA_E_OOM.
 */
pma_status pma_edge_list(const int64_t *source_index, const int64_t *target_index, int64_t nnz,
                         int64_t query_features, int64_t key_features, int add_self_loops,
                         int64_t capacity, int64_t *src_out, int64_t *tgt_out, int64_t *nnz_out);

/* Number of live edges, counting appended self-loops (kpnn2 page, attribute
   nnz); -1 for a NULL plan. */
int64_t pma_nnz(const pma_plan *plan);

/* The final edge order (given pairs, then appended loops): HOST outputs of
   pma_nnz(plan) int64 each. It is the order of the weights pma_forward
   returns (kpnn2 page, forward "Returns"). */
pma_status pma_edges(const pma_plan *plan, int64_t *src_out, int64_t *tgt_out);

/* Message for the last failed call on this thread ("" if none). */
const char *pma_last_error(void);

/* ---- inspection (tests and tools) ------------------------------------- */

typedef struct {
    int64_t query_features, key_features, embed_dim, num_heads, nnz;
    int32_t dtype;
    int32_t chunk;      /* most edges one piece of a target covers */
    int64_t n_tasks;    /* pieces: one per target, more for targets above chunk */
    int64_t n_split;    /* targets split into more than one piece */
    int64_t n_slots;    /* partial-result slots of the split targets */
    int64_t max_degree; /* largest in-degree */
    int64_t kv_rows;    /* distinct sources the edges read: the key/value rows a
                           forward projects when it skips unread sources */
} pma_info;

pma_status pma_plan_info(const pma_plan *plan, pma_info *info);

/* The plan's target-grouped edges, copied to HOST memory (blocking):
   row_ptr (L + 1), src (nnz) and eid (nnz), where row_ptr[t] counts the edges
   whose target is below t, each target's edges are ordered by ascending
   source, and eid is the entry's position in the edge order. */
pma_status pma_csr(const pma_plan *plan, int64_t *row_ptr, int64_t *src, int64_t *eid);

/* The plan's pieces, copied to HOST memory (blocking): per piece its target,
   first and end CSR position and partial slot (-1 when the target is one
   piece), ordered by (chunk - length) / 16 (longest bucket first), then
   target, then position; per
   split target its id, first slot and piece count, in ascending target
   order. A target of in-degree g has max(1, ceil(g / chunk)) pieces, piece j
   covering positions row_ptr[t] + floor(j g / n) .. row_ptr[t] + floor((j+1) g / n). */
pma_status pma_work_split(const pma_plan *plan, int64_t *task_target, int64_t *task_begin,
                          int64_t *task_end, int64_t *task_slot, int64_t *split_target,
                          int64_t *split_slot0, int64_t *split_count);

/* ---- profiling -------------------------------------------------------- */

/* Turn per-stage HIP-event timing on (1) or off (0). While on, each forward
   records events around its stages on its own stream. */
pma_status pma_profile(pma_plan *plan, int enable);

/* Time only the stages in `mask` (bit s for stage s; 0 turns timing off).
   Each timed stage adds two event records per forward on its stream, which
   themselves take some microseconds. Errors: PMA_E_NULL, PMA_E_ARG (bits
   beyond PMA_NUM_STAGES). */
pma_status pma_profile_stages(pma_plan *plan, unsigned mask);

/* Wait for the recorded events, then return per stage the summed elapsed
   milliseconds (ms[PMA_NUM_STAGES]) and launches timed (calls[PMA_NUM_STAGES])
   since the last read, and reset the sums. */
pma_status pma_profile_read(pma_plan *plan, double *ms, int64_t *calls);

/*
 * pma_gather_probe -- calibration, not part of the method. Enqueues one launch
 * that performs the loads of the edge kernel of this plan's last pma_forward
 * or pma_forward_masked: the same pieces in the same order, lane layout and
 * gather index, the plan's key/value workspace and that forward's query
 * tokens (which must still be valid), with no arithmetic beyond folding the
 * loaded words together, and one 16-byte store per (piece, sample, chunk)
 * into the plan's workspace. Its duration is what the memory path needs for
 * the edge kernel's access pattern (masks and weights left out). Errors:
 * PMA_E_NULL, PMA_E_ARG (no inference forward since the plan's workspace was
 * last allocated), PMA_E_UNSUPPORTED (head sizes the 16-byte kernel does not
 * serve; a tensor of 2 GiB or more), PMA_E_DEVICE.
 */
pma_status pma_gather_probe(pma_plan *plan, hipStream_t stream);

/*
 * pma_gather_ceiling -- calibration, not part of the method. Enqueues one
 * launch in which wavefront w gathers the 1024-byte rows rows[w * rows_per_wave
 * .. (w + 1) * rows_per_wave - 1] (the last wavefront fewer) of `table`, one
 * 16-byte chunk per lane and eight rows in flight, folds the loaded words
 * together and writes one 16-byte word per lane to sink[w * 1024 ..]. Its rate
 * over a table sized for L1, L2, the last-level cache or HBM is what the
 * vector memory path delivers for random-row gathers from that level: the
 * ceiling against which the edge kernel's gathers are read.
 *   table        DEVICE, table_bytes bytes (a multiple of 1024, under 2^32);
 *                read only
 *   rows         DEVICE int32[n_rows], row indices; an index at or past
 *                table_bytes / 1024 (or negative) reads the table's last row
 *   sink         DEVICE, ceil(n_rows / rows_per_wave) * 1024 bytes, written
 * All buffers stay the caller's. Errors: PMA_E_NULL, PMA_E_ARG (sizes out of
 * range, rows_per_wave outside [1, 2^20], more than 2^30 wavefronts),
 * PMA_E_DEVICE.
 */
pma_status pma_gather_ceiling(const void *table, uint64_t table_bytes, const int32_t *rows,
                              int64_t n_rows, int64_t rows_per_wave, void *sink,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PMA_H */
