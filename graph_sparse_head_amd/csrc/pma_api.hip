// The C ABI: plan construction, the forward pass and inspection.
// Argument checks follow the kpnn2 PackedMultiheadAttention page (constructor
// parameter table, "Raises", forward "Raises"); all of them run on the host
// before any HIP call.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>


#include "pma_internal.h"

#define PMA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

pma_status fail(pma_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

constexpr int kChunk = 256;           // shortest automatic piece length (edges)
constexpr int64_t kI32 = 2147483647;  // device edge indices are int32

struct EventPair {
    hipEvent_t a, b;
    int stage;
};

// Workspace of pma_forward_static: one file-scope device array of fixed size.
// Each GPU the library runs on holds its own copy (at its own address) from
// the module's load until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device may reach a kernel.
static_assert(PMA_STATIC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __attribute__((aligned(256))) char scratch[PMA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch`, per device ordinal

}  // namespace

struct pma_plan {
    int64_t L = 0, S = 0, E = 0, H = 0, nnz = 0;
    pma_dtype dtype = PMA_F32;
    int chunk = kChunk;
    int bchunk = kChunk;        // most edges one source piece of the backward covers
    int bsub = 1;               // PMA_BWD_SUB: target bands per XCD for the backward's source pieces
    int border = -1;            // PMA_BWD_ORDER: backward target pass over sample groups (0, 1, 2; -1 automatic)
    int bpf = -1;               // PMA_BWD_PF: backward target pass requests the next rows ahead (1), not (0), auto (-1)
    bool x3 = true;             // PMA_F32_SPLIT=0: fp32 projections on the fp32 matrix cores
    int bnt = 15;               // PMA_BWD_NT: non-temporal target-pass loads of mixed (bit 0), q and dm (bit 1), source-pass key / value loads (bit 2), dq / dk / dv stores (bit 3)
    // PMA_BWD_SORDER: banded source pass with its sample groups in turn
    // within each band (2, default) or interleaved (0)
    int bsorder = 2;
    bool batch_first_ws = false; // PMA_LAYOUT=batch: q/k/v/mixed workspace batch-first
    int xcd_map = -1;           // PMA_XCD_MAP: 1 sample group per XCD, 2 groups in turn, 0 off, -1 automatic
    bool fuse_out = true;       // PMA_FUSE_OUT=0: out_proj as a separate kernel
    bool fuse_in = true;        // PMA_FUSE_IN=0: q projection as a separate kernel
    int nt = -1;                // PMA_NT: non-temporal streams (bit 0 q loads, bit 1 mixed / out stores), auto (-1)
    int persist = -1;           // PMA_PERSIST: edge-kernel workgroups per CU (0: one per piece, -1 auto)
    int compact = -1;           // PMA_COMPACT: key/value rows only for read sources (1), all (0), auto (-1)
    bool hot = false;           // PMA_HOT=1: hot-row cache in the q-projecting edge kernel
    int coop = 0;               // PMA_COOP=1: split targets merged inside the edge kernel
    // hot-row cache: the gather index (hot_key) with ~slot for the edges of
    // the n_hot most-read rows hot_src[slot]
    int32_t *hot_csr = nullptr, *hot_src = nullptr;
    const int32_t *hot_key = nullptr;
    int n_hot = 0;
    std::vector<int64_t> h_src, h_tgt;
    pma::GraphDev g;
    // workspace, grown on demand
    int64_t ws_B = 0;
    bool ws_weights = false;
    void *qt = nullptr, *kv = nullptr, *mixed = nullptr;
    float *part_acc = nullptr, *part_ml = nullptr, *stat_ml = nullptr, *scores = nullptr;
    uint64_t *kpm_bits = nullptr;   // key_padding_mask packed by source
    uint32_t *kpm_csr = nullptr;    // the same by CSR position (32-bit words)
    // backward and PackedLinear scratch, grown on demand
    char *bw = nullptr;
    size_t bw_bytes = 0;
    char *lin = nullptr;
    size_t lin_bytes = 0;
    // the edge-kernel arguments of the last inference forward (for
    // pma_gather_probe); probe_ok is cleared when the workspace is reallocated
    pma::EdgeArgs probe_ea;
    bool probe_ok = false;
    // profiling
    unsigned prof = 0;   // stages timed: bit s for stage s
    std::vector<EventPair> pending;
    std::vector<hipEvent_t> pool;
    double ms[PMA_NUM_STAGES] = {0};
    int64_t calls[PMA_NUM_STAGES] = {0};
};

namespace {

void free_workspace(pma_plan *p)
{
    void *ptrs[] = {p->qt,     p->kv,      p->mixed,  p->part_acc,
                    p->part_ml, p->stat_ml, p->scores, p->kpm_bits, p->kpm_csr};
    for (void *q : ptrs)
        if (q)
            (void)hipFree(q);
    p->qt = p->kv = p->mixed = nullptr;
    p->part_acc = p->part_ml = p->stat_ml = p->scores = nullptr;
    p->kpm_bits = nullptr;
    p->kpm_csr = nullptr;
    p->ws_B = 0;
    p->ws_weights = false;
    p->probe_ok = false;
}

// Buffers for a batch of B: q, keys/values, mixed, the split partials and
// the packed key_padding_mask; scores and final (max, sum) only for
// need_weights.
pma_status ensure_workspace(pma_plan *p, int64_t B, bool weights, hipStream_t s)
{
    if (B <= p->ws_B && (!weights || p->ws_weights))
        return PMA_OK;
    const int64_t nB = B > p->ws_B ? B : p->ws_B;
    const bool nw = weights || p->ws_weights;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return fail(PMA_E_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
    free_workspace(p);
    const size_t es = p->dtype == PMA_BF16 ? 2 : 4;
    const size_t slots = (size_t)(p->g.n_slots > 0 ? p->g.n_slots : 1);
    struct {
        void **ptr;
        size_t bytes;
    } want[] = {
        {&p->qt, (size_t)p->L * nB * p->E * es},
        {&p->kv, (size_t)p->S * 2 * nB * p->E * es},
        {&p->mixed, (size_t)p->L * nB * p->E * es},
        {(void **)&p->part_acc, slots * nB * p->E * 4},
        {(void **)&p->part_ml, slots * nB * p->H * 2 * 4},
        {(void **)&p->stat_ml, nw ? (size_t)p->L * nB * p->H * 2 * 4 : 0},
        {(void **)&p->scores, nw ? (size_t)p->nnz * nB * p->H * 4 : 0},
        {(void **)&p->kpm_bits, (size_t)p->S * ((nB + 63) / 64) * 8},
        // (+ 4 positions: the backward reads mask words 4 edges at a time)
        {(void **)&p->kpm_csr, (size_t)(p->nnz + 4) * ((nB + 31) / 32) * 4},
    };
    for (auto &w : want) {
        if (w.bytes == 0)
            continue;
        e = hipMalloc(w.ptr, w.bytes);
        if (e != hipSuccess) {
            free_workspace(p);
            return fail(e == hipErrorOutOfMemory ? PMA_E_OOM : PMA_E_DEVICE,
                        "workspace allocation of %zu bytes: %s", w.bytes, hipGetErrorString(e));
        }
    }
    p->ws_B = nB;
    p->ws_weights = nw;
    return PMA_OK;
}

hipEvent_t take_event(pma_plan *p)
{
    if (!p->pool.empty()) {
        hipEvent_t ev = p->pool.back();
        p->pool.pop_back();
        return ev;
    }
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess)
        return nullptr;
    return ev;
}

struct StageTimer {
    pma_plan *p;
    hipStream_t s;
    bool off = false;   // no events at all (the allocation-free forward)
    EventPair cur{nullptr, nullptr, -1};
    void begin(int stage)
    {
        if (off || !((p->prof >> stage) & 1u))
            return;
        cur.a = take_event(p);
        cur.b = take_event(p);
        cur.stage = stage;
        if (cur.a)
            (void)hipEventRecord(cur.a, s);
    }
    void end()
    {
        if (off || !p->prof || cur.stage < 0)
            return;
        if (cur.a && cur.b) {
            (void)hipEventRecord(cur.b, s);
            p->pending.push_back(cur);
        }
        cur.stage = -1;
    }
};

}  // namespace

PMA_API const char *pma_last_error(void) { return g_err; }

namespace {

// attn: a plan for the attention calls (embed_dim, num_heads checked); else
// a graph-only plan (embed_dim = num_heads = 0) for the PackedLinear calls.
// The hot-row cache of the q-projecting edge kernel: the kHotRows rows of the
// gather index idx (rows rows) that the most edges read, if read by at least
// two, become LDS slots; hot_csr is idx with ~slot in their place. Built once
// per index array (host pass over the nnz indices).
pma_status build_hot(pma_plan *p, const int32_t *idx, int64_t rows, hipStream_t stream)
{
    if (p->hot_key == idx)
        return PMA_OK;
    const int64_t nnz = p->nnz;
    std::vector<int32_t> h, order, slot_of;
    try {
        h.resize(nnz + pma::kSrcPad, 0);
        order.resize(rows);
        slot_of.assign(rows, -1);
    } catch (...) {
        return PMA_E_OOM;
    }
    if (hipMemcpyAsync(h.data(), idx, nnz * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return PMA_E_DEVICE;
    std::vector<int64_t> cnt(rows, 0);
    for (int64_t i = 0; i < nnz; ++i)
        ++cnt[h[i]];
    std::iota(order.begin(), order.end(), 0);
    const int64_t k = std::min<int64_t>(pma::kHotRows, rows);
    std::partial_sort(order.begin(), order.begin() + k, order.end(), [&](int32_t a, int32_t b) {
        return cnt[a] > cnt[b] || (cnt[a] == cnt[b] && a < b);
    });
    int n = 0;
    while (n < k && cnt[order[n]] >= 2)
        ++n;
    for (int i = 0; i < n; ++i)
        slot_of[order[i]] = i;
    for (int64_t i = 0; i < nnz; ++i)
        if (slot_of[h[i]] >= 0)
            h[i] = ~slot_of[h[i]];
    // each target row lists its cached sources first (the edges of a row may
    // come in any order: the softmax and the mix are sums over them)
    std::vector<int32_t> rp;
    try {
        rp.resize(p->L + 1);
    } catch (...) {
        return PMA_E_OOM;
    }
    if (hipMemcpyAsync(rp.data(), p->g.row_ptr, (p->L + 1) * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return PMA_E_DEVICE;
    for (int64_t t = 0; t < p->L; ++t)
        std::stable_partition(h.begin() + rp[t], h.begin() + rp[t + 1], [](int32_t v) { return v < 0; });
    if (!p->hot_csr && hipMalloc(&p->hot_csr, (nnz + pma::kSrcPad) * sizeof(int32_t)) != hipSuccess)
        return PMA_E_OOM;
    if (!p->hot_src && hipMalloc(&p->hot_src, pma::kHotRows * sizeof(int32_t)) != hipSuccess)
        return PMA_E_OOM;
    order.resize(pma::kHotRows, 0);
    if (hipMemcpyAsync(p->hot_csr, h.data(), (nnz + pma::kSrcPad) * sizeof(int32_t), hipMemcpyHostToDevice,
                       stream) != hipSuccess ||
        hipMemcpyAsync(p->hot_src, order.data(), pma::kHotRows * sizeof(int32_t), hipMemcpyHostToDevice,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return PMA_E_DEVICE;
    p->hot_key = idx;
    p->n_hot = n;
    return PMA_OK;
}

// The constructor's index rules on the host (kpnn2 page, constructor
// parameter table and "Raises"): nnz >= 1, indices present and in range,
// add_self_loops only with L == S; then the edge order: the given pairs, and
// with add_self_loops every missing (i, i) after them in ascending i. Sizes
// are checked by the caller. Repeated pairs are left to the caller
// (pma_create finds them on the device after sorting; pma_edge_list on the
// host).
pma_status host_edges(const int64_t *source_index, const int64_t *target_index, int64_t nnz,
                      int64_t L, int64_t S, int add_self_loops, std::vector<int64_t> &src,
                      std::vector<int64_t> &tgt)
{
    if (nnz < 1)
        return fail(PMA_E_INDEX_EMPTY, "the indices are empty (nnz = %lld)", (long long)nnz);
    if (!source_index || !target_index)
        return fail(PMA_E_NULL, "source_index or target_index is NULL");
    if (add_self_loops && L != S)
        return fail(PMA_E_SELF_LOOPS,
                    "add_self_loops needs query_features == key_features (%lld != %lld)",
                    (long long)L, (long long)S);
    for (int64_t i = 0; i < nnz; ++i) {
        if (source_index[i] < 0 || source_index[i] >= S)
            return fail(PMA_E_INDEX_RANGE, "source_index[%lld] = %lld outside [0, %lld)",
                        (long long)i, (long long)source_index[i], (long long)S);
        if (target_index[i] < 0 || target_index[i] >= L)
            return fail(PMA_E_INDEX_RANGE, "target_index[%lld] = %lld outside [0, %lld)",
                        (long long)i, (long long)target_index[i], (long long)L);
    }
    try {
        src.assign(source_index, source_index + nnz);
        tgt.assign(target_index, target_index + nnz);
        if (add_self_loops) {
            std::vector<char> has(L, 0);
            for (int64_t i = 0; i < nnz; ++i)
                if (source_index[i] == target_index[i])
                    has[source_index[i]] = 1;
            for (int64_t i = 0; i < L; ++i)
                if (!has[i]) {
                    src.push_back(i);
                    tgt.push_back(i);
                }
        }
    } catch (...) {
        return fail(PMA_E_OOM, "host allocation failed");
    }
    return PMA_OK;
}

pma_status create_impl(pma_plan **plan, const int64_t *source_index, const int64_t *target_index,
                       int64_t nnz, int64_t query_features, int64_t key_features,
                       int64_t embed_dim, int64_t num_heads, int add_self_loops, pma_dtype dtype,
                       hipStream_t stream, bool attn)
{
    g_err[0] = 0;
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    *plan = nullptr;
    if (dtype != PMA_F32 && dtype != PMA_BF16)
        return fail(PMA_E_DTYPE, "dtype %d is not PMA_F32 or PMA_BF16", (int)dtype);
    if (add_self_loops != 0 && add_self_loops != 1)
        return fail(PMA_E_ARG, "add_self_loops must be 0 or 1");
    const int64_t L = query_features, S = key_features, E = embed_dim, H = num_heads;
    if (L <= 0 || S <= 0 || (attn && (E <= 0 || H <= 0)))
        return fail(PMA_E_SIZE, "sizes must be positive (L=%lld S=%lld E=%lld H=%lld)",
                    (long long)L, (long long)S, (long long)E, (long long)H);
    if (attn && E % H != 0)
        return fail(PMA_E_SIZE, "embed_dim %lld is not divisible by num_heads %lld",
                    (long long)E, (long long)H);
    if (L > kI32 || S > kI32 || nnz > kI32)
        return fail(PMA_E_UNSUPPORTED, "more than 2^31 - 1 edges or tokens");

    pma_plan *p = new (std::nothrow) pma_plan;
    if (!p)
        return fail(PMA_E_OOM, "host allocation failed");
    {
        // (repeated pairs are found on the device after the sort, below)
        const pma_status st = host_edges(source_index, target_index, nnz, L, S, add_self_loops,
                                         p->h_src, p->h_tgt);
        if (st != PMA_OK) {
            delete p;
            return st;
        }
    }
    p->L = L;
    p->S = S;
    p->E = E;
    p->H = H;
    p->nnz = (int64_t)p->h_src.size();
    p->dtype = dtype;
    // Tuning knobs, read once per plan (defaults are the measured best):
    //   PMA_CHUNK      most edges per piece of a target (1..65535; default
    //                  automatic, see below)
    //   PMA_FUSE_OUT   0: out_proj as a separate kernel
    //   PMA_FUSE_IN    0: q projection as a separate kernel
    //   PMA_XCD_MAP    1: one sample group per XCD, 2: sample groups in
    //                  turn, 0: interleaved (default automatic)
    //   PMA_NT         0..3: non-temporal q loads (bit 0) and mixed / out
    //                  stores (bit 1)
    //   PMA_LAYOUT     "batch": batch-first q / k / v / mixed workspace
    //   PMA_PERSIST    n: at most n edge-kernel workgroups per CU, each
    //                  wavefront walking several pieces (0: one per piece)
    //   PMA_COMPACT    1 / 0: force or forbid projecting keys and values only
    //                  for the sources some edge reads
    //   PMA_BWD_CHUNK  n: most edges of one source piece in the backward pass
    //   PMA_BWD_SUB    n: target bands per XCD for those pieces (1..64)
    //   PMA_BWD_ORDER  backward target pass over sample groups, as PMA_XCD_MAP
    //   PMA_BWD_PF     1 / 0: backward target pass with or without the next
    //                  rows requested ahead (default automatic)
    //   PMA_BWD_SORDER 0: banded source pass with its sample groups
    //                  interleaved instead of in turn within each band
    //   PMA_F32_SPLIT  0: fp32 projections at embed_dim 128 on the fp32
    //                  matrix cores instead of split-bf16 products (proj_x3;
    //                  bipartite key/value projection 206 -> 2 x 90 us)
    //   PMA_BWD_NT     0..15: non-temporal backward streams, each read or
    //                  written once there: the target pass's mixed rows (bit
    //                  0) and q and dm rows (bit 1), the source pass's own
    //                  key and value rows (bit 2), the dq, dk, dv stores (bit
    //                  3); default 15 (training step, cold: gene 0.887 ->
    //                  0.866 ms, 100k-node 5.54 -> 5.48, bipartite 1.84 -> 1.80)
    //   PMA_HOT        1: hot-row LDS cache in the q-projecting edge kernel
    //   PMA_COOP       1: merge split targets of at most 4 pieces in the edge
    //                  kernel's leading workgroups (one per target and sample
    //                  group) instead of a launch of their own; measured
    //                  on MI355X 2-3 us slower on the gene-regulatory forward
    // Piece length: a target is split only when it has far more edges than
    // the average target (16x, rounded up to a power of two, at least 256).
    // Splitting balances graphs with a few very long rows among many short
    // ones; where rows are uniformly long, whole rows avoid the partial
    // results and the merge (measured on MI355X: gene-like graphs best at
    // 256, pathway maps with up to 500 members per row best unsplit).
    {
        const double avg = (double)p->nnz / (double)L;
        int c = kChunk;
        while (c < 65536 && c < 16.0 * avg)
            c <<= 1;
        p->chunk = c > 65535 ? 65535 : c;
    }
    if (const char *ev = getenv("PMA_CHUNK")) {
        const long c = strtol(ev, nullptr, 10);
        if (c >= 1 && c <= 65535)
            p->chunk = (int)c;
    }
    if (const char *ev = getenv("PMA_BWD_CHUNK")) {
        const long c = strtol(ev, nullptr, 10);
        if (c >= 1 && c <= 65535)
            p->bchunk = (int)c;
    }
    if (const char *ev = getenv("PMA_BWD_SORDER"))
        p->bsorder = ev[0] == '0' ? 0 : 2;
    if (const char *ev = getenv("PMA_BWD_PF"))
        p->bpf = ev[0] == '0' ? 0 : 1;
    if (const char *ev = getenv("PMA_F32_SPLIT"))
        p->x3 = ev[0] != '0';
    if (const char *ev = getenv("PMA_BWD_NT")) {
        const long v = strtol(ev, nullptr, 10);
        if (v >= 0 && v <= 15)
            p->bnt = (int)v;
    }
    if (const char *ev = getenv("PMA_BWD_ORDER"))
        p->border = ev[0] == '1' ? 1 : ev[0] == '2' ? 2 : 0;
    if (const char *ev = getenv("PMA_BWD_SUB")) {
        const long c = strtol(ev, nullptr, 10);
        if (c >= 1 && c <= 64)
            p->bsub = (int)c;
    }
    if (const char *ev = getenv("PMA_FUSE_OUT"))
        p->fuse_out = ev[0] != '0';
    if (const char *ev = getenv("PMA_HOT"))
        p->hot = ev[0] == '1';
    if (const char *ev = getenv("PMA_COOP"))
        p->coop = ev[0] == '1' ? 1 : 0;
    if (const char *ev = getenv("PMA_FUSE_IN"))
        p->fuse_in = ev[0] != '0';
    if (const char *ev = getenv("PMA_XCD_MAP"))
        p->xcd_map = ev[0] == '0' ? 0 : ev[0] == '2' ? 2 : 1;
    if (const char *ev = getenv("PMA_NT")) {
        const long v = strtol(ev, nullptr, 10);
        if (v >= 0 && v <= 3)
            p->nt = (int)v;
    }
    if (const char *ev = getenv("PMA_LAYOUT"))
        p->batch_first_ws = strcmp(ev, "batch") == 0;
    if (const char *ev = getenv("PMA_COMPACT"))
        p->compact = ev[0] == '0' ? 0 : 1;
    if (const char *ev = getenv("PMA_PERSIST")) {
        const long c = strtol(ev, nullptr, 10);
        if (c >= 0 && c <= 64)
            p->persist = (int)c;
    }
    if (p->nnz + L > kI32) {
        delete p;
        return fail(PMA_E_UNSUPPORTED, "nnz + query_features exceeds 2^31 - 1");
    }
    std::vector<int32_t> s32, t32;
    try {
        s32.resize(p->nnz);
        t32.resize(p->nnz);
    } catch (...) {
        delete p;
        return fail(PMA_E_OOM, "host allocation failed");
    }
    for (int64_t i = 0; i < p->nnz; ++i) {
        s32[i] = (int32_t)p->h_src[i];
        t32[i] = (int32_t)p->h_tgt[i];
    }
    char err[256] = "";
    pma_status st = pma::build_graph(s32.data(), t32.data(), p->nnz, L, S, p->chunk, stream,
                                     &p->g, err, sizeof err);
    if (st != PMA_OK) {
        delete p;
        return fail(st, "%s", err);
    }
    *plan = p;
    return PMA_OK;
}

}  // namespace

PMA_API pma_status pma_create(pma_plan **plan, const int64_t *source_index,
                              const int64_t *target_index, int64_t nnz, int64_t query_features,
                              int64_t key_features, int64_t embed_dim, int64_t num_heads,
                              int add_self_loops, pma_dtype dtype, hipStream_t stream)
{
    return create_impl(plan, source_index, target_index, nnz, query_features, key_features,
                       embed_dim, num_heads, add_self_loops, dtype, stream, true);
}

PMA_API pma_status pma_create_graph(pma_plan **plan, const int64_t *source_index,
                                    const int64_t *target_index, int64_t nnz,
                                    int64_t query_features, int64_t key_features,
                                    int add_self_loops, pma_dtype dtype, hipStream_t stream)
{
    return create_impl(plan, source_index, target_index, nnz, query_features, key_features, 0, 0,
                       add_self_loops, dtype, stream, false);
}

PMA_API pma_status pma_destroy(pma_plan *plan)
{
    if (!plan)
        return PMA_OK;
    (void)hipDeviceSynchronize();
    pma::free_graph(&plan->g);
    free_workspace(plan);
    if (plan->hot_csr)
        (void)hipFree(plan->hot_csr);
    if (plan->hot_src)
        (void)hipFree(plan->hot_src);
    if (plan->bw)
        (void)hipFree(plan->bw);
    if (plan->lin)
        (void)hipFree(plan->lin);
    for (auto &ev : plan->pending) {
        (void)hipEventDestroy(ev.a);
        (void)hipEventDestroy(ev.b);
    }
    for (hipEvent_t ev : plan->pool)
        (void)hipEventDestroy(ev);
    delete plan;
    return PMA_OK;
}

PMA_API pma_status pma_edge_list(const int64_t *source_index, const int64_t *target_index,
                                 int64_t nnz, int64_t query_features, int64_t key_features,
                                 int add_self_loops, int64_t capacity, int64_t *src_out,
                                 int64_t *tgt_out, int64_t *nnz_out)
{
    g_err[0] = 0;
    if (!nnz_out)
        return fail(PMA_E_NULL, "nnz_out is NULL");
    *nnz_out = 0;
    if (add_self_loops != 0 && add_self_loops != 1)
        return fail(PMA_E_ARG, "add_self_loops must be 0 or 1");
    const int64_t L = query_features, S = key_features;
    if (L <= 0 || S <= 0)
        return fail(PMA_E_SIZE, "sizes must be positive (L=%lld S=%lld)", (long long)L,
                    (long long)S);
    if (L > kI32 || S > kI32 || nnz > kI32)
        return fail(PMA_E_UNSUPPORTED, "more than 2^31 - 1 edges or tokens");
    std::vector<int64_t> src, tgt;
    pma_status st = host_edges(source_index, target_index, nnz, L, S, add_self_loops, src, tgt);
    if (st != PMA_OK)
        return st;
    // repeated pairs: sort (target, source) keys, compare neighbours; the
    // appended loops are never repeats (only missing ones are appended)
    {
        std::vector<int64_t> key;
        try {
            key.resize(nnz);
        } catch (...) {
            return fail(PMA_E_OOM, "host allocation failed");
        }
        for (int64_t i = 0; i < nnz; ++i)
            key[i] = target_index[i] * S + source_index[i];
        std::sort(key.begin(), key.end());
        for (int64_t i = 1; i < nnz; ++i)
            if (key[i] == key[i - 1])
                return fail(PMA_E_INDEX_DUPLICATE, "the pair (source %lld, target %lld) repeats",
                            (long long)(key[i] % S), (long long)(key[i] / S));
    }
    const int64_t n = (int64_t)src.size();
    *nnz_out = n;
    if (capacity < n)
        return fail(PMA_E_SIZE, "the edge list has %lld entries, capacity is %lld", (long long)n,
                    (long long)capacity);
    if (!src_out || !tgt_out)
        return fail(PMA_E_NULL, "src_out or tgt_out is NULL");
    memcpy(src_out, src.data(), n * sizeof(int64_t));
    memcpy(tgt_out, tgt.data(), n * sizeof(int64_t));
    return PMA_OK;
}

PMA_API int64_t pma_nnz(const pma_plan *plan) { return plan ? plan->nnz : -1; }

PMA_API pma_status pma_edges(const pma_plan *plan, int64_t *src_out, int64_t *tgt_out)
{
    if (!plan || !src_out || !tgt_out)
        return fail(PMA_E_NULL, "NULL argument");
    memcpy(src_out, plan->h_src.data(), plan->nnz * sizeof(int64_t));
    memcpy(tgt_out, plan->h_tgt.data(), plan->nnz * sizeof(int64_t));
    return PMA_OK;
}

PMA_API pma_status pma_plan_info(const pma_plan *plan, pma_info *info)
{
    if (!plan || !info)
        return fail(PMA_E_NULL, "NULL argument");
    info->query_features = plan->L;
    info->key_features = plan->S;
    info->embed_dim = plan->E;
    info->num_heads = plan->H;
    info->nnz = plan->nnz;
    info->dtype = (int32_t)plan->dtype;
    info->chunk = plan->chunk;
    info->n_tasks = plan->g.n_tasks;
    info->n_split = plan->g.n_split;
    info->n_slots = plan->g.n_slots;
    info->max_degree = plan->g.max_degree;
    info->kv_rows = plan->g.n_kv;
    return PMA_OK;
}

namespace {

pma_status copy_widen(const int32_t *dev, int64_t n, int64_t *host)
{
    if (n <= 0)
        return PMA_OK;
    std::vector<int32_t> tmp(n);
    hipError_t e = hipMemcpy(tmp.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(PMA_E_DEVICE, "hipMemcpy: %s", hipGetErrorString(e));
    for (int64_t i = 0; i < n; ++i)
        host[i] = tmp[i];
    return PMA_OK;
}

}  // namespace

PMA_API pma_status pma_csr(const pma_plan *plan, int64_t *row_ptr, int64_t *src, int64_t *eid)
{
    if (!plan || !row_ptr || !src || !eid)
        return fail(PMA_E_NULL, "NULL argument");
    pma_status st = copy_widen(plan->g.row_ptr, plan->L + 1, row_ptr);
    if (st == PMA_OK)
        st = copy_widen(plan->g.csr_src, plan->nnz, src);
    if (st == PMA_OK)
        st = copy_widen(plan->g.csr_eid, plan->nnz, eid);
    return st;
}

PMA_API pma_status pma_work_split(const pma_plan *plan, int64_t *task_target,
                                  int64_t *task_begin, int64_t *task_end, int64_t *task_slot,
                                  int64_t *split_target, int64_t *split_slot0,
                                  int64_t *split_count)
{
    if (!plan || !task_target || !task_begin || !task_end || !task_slot ||
        (plan->g.n_split > 0 && (!split_target || !split_slot0 || !split_count)))
        return fail(PMA_E_NULL, "NULL argument");
    const pma::GraphDev &g = plan->g;
    pma_status st = copy_widen(g.task_target, g.n_tasks, task_target);
    if (st == PMA_OK) st = copy_widen(g.task_begin, g.n_tasks, task_begin);
    if (st == PMA_OK) st = copy_widen(g.task_end, g.n_tasks, task_end);
    if (st == PMA_OK) st = copy_widen(g.task_slot, g.n_tasks, task_slot);
    if (st == PMA_OK) st = copy_widen(g.split_target, g.n_split, split_target);
    if (st == PMA_OK) st = copy_widen(g.split_slot0, g.n_split, split_slot0);
    if (st == PMA_OK) st = copy_widen(g.split_count, g.n_split, split_count);
    return st;
}

namespace {

// Byte offsets of the training save area: q (B, L, E), k then v (B, S, E),
// mixed (B, L, E) in the plan's dtype, softmax (max, sum) [L][B][H][2] fp32.
struct SaveLayout {
    size_t q, k, v, mixed, ml, total;
};

// Whether a training forward projects keys and values only for the sources
// some edge reads (then the save area holds n_kv key/value rows per sample).
bool train_compact(const pma_plan *p)
{
    return p->g.n_kv < p->S && p->compact != 0;
}

SaveLayout save_layout(const pma_plan *p, int64_t B)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t es = p->dtype == PMA_BF16 ? 2 : 4;
    SaveLayout s;
    s.q = 0;
    s.k = up(s.q + (size_t)B * p->L * p->E * es);
    s.v = s.k + (size_t)B * p->S * p->E * es;
    s.mixed = up(s.v + (size_t)B * p->S * p->E * es);
    s.ml = up(s.mixed + (size_t)B * p->L * p->E * es);
    s.total = up(s.ml + (size_t)p->L * B * p->H * 2 * 4);
    return s;
}

// The workspace pointers one forward uses (see ensure_workspace).
struct Ws {
    void *qt, *kv, *mixed;
    float *part_acc, *part_ml, *stat_ml, *scores;
};

// Device address of the static scratch on the current device, looked up once
// per device (with that device current) and kept.
pma_status static_scratch(char **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(PMA_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PMA_E_UNSUPPORTED, "device ordinal %d beyond the static scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !a)
            return fail(PMA_E_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch[dev] = a;
    }
    *ptr = static_cast<char *>(g_scratch[dev]);
    return PMA_OK;
}

// The allocation-free forward's workspace, carved from the static scratch in
// 256-byte aligned pieces: q (unless projected inside the edge kernel), the
// S_ws key/value rows, mixed (unless out_proj is fused), the partial results
// of split targets and, with need_weights, the softmax statistics and scores.
// Every piece is written before it is read within the forward, so nothing is
// cleared. Fails with PMA_E_SIZE, before any launch, beyond the scratch size.
pma_status carve_static(const pma_plan *p, int64_t B, int64_t S_ws, bool need_q, bool need_mixed,
                        bool weights, Ws *w)
{
    const size_t es = p->dtype == PMA_BF16 ? 2 : 4;
    const size_t slots = (size_t)(p->g.n_slots > 0 ? p->g.n_slots : 1);
    const size_t rows = (size_t)p->L * B * p->E * es;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t o_q = need_q ? take(rows) : 0;
    const size_t o_kv = take((size_t)S_ws * 2 * B * p->E * es);
    const size_t o_mixed = need_mixed ? take(rows) : 0;
    const size_t o_pacc = take(slots * B * p->E * 4);
    const size_t o_pml = take(slots * B * p->H * 2 * 4);
    const size_t o_stat = weights ? take((size_t)p->L * B * p->H * 2 * 4) : 0;
    const size_t o_sc = weights ? take((size_t)p->nnz * B * p->H * 4) : 0;
    if (off > PMA_STATIC_SCRATCH_BYTES)
        return fail(PMA_E_SIZE,
                    "this forward needs %zu bytes of workspace; the allocation-free forward's "
                    "static scratch holds %zu",
                    off, (size_t)PMA_STATIC_SCRATCH_BYTES);
    char *base = nullptr;
    const pma_status st = static_scratch(&base);
    if (st != PMA_OK)
        return st;
    w->qt = need_q ? base + o_q : nullptr;
    w->kv = base + o_kv;
    w->mixed = need_mixed ? base + o_mixed : nullptr;
    w->part_acc = reinterpret_cast<float *>(base + o_pacc);
    w->part_ml = reinterpret_cast<float *>(base + o_pml);
    w->stat_ml = weights ? reinterpret_cast<float *>(base + o_stat) : nullptr;
    w->scores = weights ? reinterpret_cast<float *>(base + o_sc) : nullptr;
    return PMA_OK;
}

pma_status forward_impl(pma_plan *plan, int64_t batch, const void *query, const void *key,
                        const void *value, const void *q_w, const void *q_b, const void *k_w,
                        const void *k_b, const void *v_w, const void *v_b, const void *o_w,
                        const void *o_b, void *out, float *weights, int average_attn_weights,
                        const uint8_t *kpm, int kpm_per_sample, char *save, bool no_alloc,
                        hipStream_t stream)
{
    g_err[0] = 0;
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    if (plan->E == 0)
        return fail(PMA_E_ARG, "the plan has no attention sizes (made by pma_create_graph)");
    if (batch <= 0)
        return fail(PMA_E_SIZE, "batch must be positive (got %lld)", (long long)batch);
    if (!query || !key || !value || !q_w || !k_w || !v_w || !o_w || !out)
        return fail(PMA_E_NULL, "a token, weight or output pointer is NULL");
    const int nb = (q_b != nullptr) + (k_b != nullptr) + (v_b != nullptr) + (o_b != nullptr);
    if (nb != 0 && nb != 4)
        return fail(PMA_E_ARG, "biases must be all given or all NULL");
    if (average_attn_weights != 0 && average_attn_weights != 1)
        return fail(PMA_E_ARG, "average_attn_weights must be 0 or 1");
    pma_plan *p = plan;
    const int64_t B = batch, L = p->L, S = p->S, E = p->E;
    if ((L > S ? L : S) * B * 2 * E > ((int64_t)1 << 40))
        return fail(PMA_E_UNSUPPORTED, "batch too large for one forward");
    if (no_alloc && (kpm || save))
        return fail(PMA_E_ARG, "the allocation-free forward takes no mask and no save area");
    pma_status st = PMA_OK;
    StageTimer tm{p, stream};
    tm.off = no_alloc;
    const size_t es = p->dtype == PMA_BF16 ? 2 : 4;
    // Keys and values are needed only for the sources some edge reads
    // (n_kv of S). Projecting just those rows saves work unless query, key
    // and value are one tensor and most sources are read: then one pass over
    // the tokens that writes q, k and v at once moves fewer bytes (a separate
    // key/value pass re-reads n_kv / S of the tokens; it pays below 3/5).
    // A training forward decides from the plan alone (train_compact), so that
    // the backward reads the saved keys and values the same way.
    const bool shared = query == key && key == value && L == S;
    const int64_t n_kv = p->g.n_kv;
    const bool compact = save ? train_compact(p)
                              : n_kv < S && (p->compact >= 0 ? p->compact == 1
                                                              : (!shared || 5 * n_kv < 3 * S));
    const int64_t S_ws = compact ? n_kv : S;   // key/value rows in the workspace
    const pma::Layout lay = pma::make_layout(save ? true : p->batch_first_ws, B, L, S_ws, E);

    // out_proj in the edge / merge epilogue where it applies (16-byte aligned
    // Wo and out), and then also the q projection in the edge kernel's
    // prologue (16-byte aligned Wq and query): q never goes to memory.
    const bool fuse_out = !save && p->fuse_out && pma::out_fusable(E, p->H, p->dtype) &&
                          (((uintptr_t)o_w | (uintptr_t)out) & 15) == 0;
    const bool fuse_in = fuse_out && p->fuse_in && pma::q_fusable(E, p->H, p->dtype) &&
                         (((uintptr_t)q_w | (uintptr_t)query) & 15) == 0;

    // Workspace: the plan's (grown on demand), or for the allocation-free
    // forward carved from the static scratch array, only what this call uses.
    Ws w;
    if (no_alloc) {
        st = carve_static(p, B, S_ws, !fuse_in, !fuse_out, weights != nullptr, &w);
    } else {
        st = ensure_workspace(p, B, weights != nullptr, stream);
        w = {p->qt, p->kv, p->mixed, p->part_acc, p->part_ml, p->stat_ml, p->scores};
    }
    if (st != PMA_OK)
        return st;
    // With a save area (training) q, k, v, mixed and the softmax statistics
    // go there, batch-first, for pma_backward; otherwise to the workspace.
    const SaveLayout sv = save_layout(p, B);
    void *qt = save ? (void *)(save + sv.q) : w.qt;
    char *kvc = save ? save + sv.k : static_cast<char *>(w.kv);
    void *mixed_ws = save ? (void *)(save + sv.mixed) : w.mixed;

    // Step 1: q, k, v projections into the workspace layout. Caller tokens are
    // batch-first and read in storage order (key/value rows through the list
    // of read sources when compact).
    tm.begin(PMA_STAGE_PROJ_IN);
    const pma::ProjOut oq{q_w, q_b, qt, lay.q_b, lay.q_t};
    const pma::ProjOut ok{k_w, k_b, kvc, lay.kv_b, lay.kv_s};
    const pma::ProjOut ov{v_w, v_b, kvc + (size_t)lay.kv_v * es, lay.kv_b, lay.kv_s};
    auto in_args = [&](const void *x, int64_t n, int nblk, pma::ProjOut o0, pma::ProjOut o1,
                       pma::ProjOut o2) {
        pma::ProjArgs a{x, B * n, n, B, 0, nblk, {o0, o1, o2}};
        a.x_token_major = 0;
        a.x3 = p->x3 && p->dtype == PMA_F32;
        return a;
    };
    auto kv_args = [&](const void *x, int nblk, pma::ProjOut o0, pma::ProjOut o1) {
        pma::ProjArgs a = in_args(x, S_ws, nblk, o0, o1, o1);
        if (compact) {
            a.row_list = p->g.kv_rows;
            a.n_in = S;
        }
        return a;
    };
    if (shared && !compact && !fuse_in) {
        st = pma::launch_proj(in_args(query, L, 3, oq, ok, ov), E, p->dtype, stream);
    } else {
        if (!fuse_in)
            st = pma::launch_proj(in_args(query, L, 1, oq, oq, oq), E, p->dtype, stream);
        if (st == PMA_OK && key == value) {
            st = pma::launch_proj(kv_args(key, 2, ok, ov), E, p->dtype, stream);
        } else if (st == PMA_OK) {
            st = pma::launch_proj(kv_args(key, 1, ok, ok), E, p->dtype, stream);
            if (st == PMA_OK)
                st = pma::launch_proj(kv_args(value, 1, ov, ov), E, p->dtype, stream);
        }
    }
    tm.end();
    if (st != PMA_OK)
        return fail(st, "projection launch failed: %s", hipGetErrorString(hipGetLastError()));

    pma::EdgeArgs ea;
    ea.g = &p->g;
    ea.gather_src = compact ? p->g.csr_kv : p->g.csr_src;
    ea.B = B;
    ea.L = L;
    ea.S = S;
    ea.E = E;
    ea.H = p->H;
    ea.nnz = p->nnz;
    ea.dt = p->dtype;
    ea.lay = lay;
    ea.qt = qt;
    if (fuse_in) {   // the edge kernel reads the caller's (B, L, E) query rows
        ea.qt = query;
        ea.lay.q_t = E;
        ea.lay.q_b = L * E;
    }
    ea.kv = kvc;
    ea.kv_bytes = (uint64_t)S_ws * 2 * B * E * es;
    ea.mixed = mixed_ws;
    ea.part_acc = w.part_acc;
    ea.part_ml = w.part_ml;
    ea.stat_ml = save ? reinterpret_cast<float *>(save + sv.ml) : (weights ? w.stat_ml : nullptr);
    ea.scores = weights ? w.scores : nullptr;
    ea.weights = weights;
    ea.average = average_attn_weights;
    if (kpm) {
        st = pma::pack_mask(kpm, kpm_per_sample ? S : 0, B, S, p->kpm_bits, stream);
        if (st != PMA_OK)
            return fail(st, "mask packing failed: %s", hipGetErrorString(hipGetLastError()));
        ea.kpm_bits = p->kpm_bits;
        ea.kpm_words = (int)((B + 63) / 64);
        ea.kpm_w32 = (int)((B + 31) / 32);
        st = pma::gather_mask(p->kpm_bits, ea.kpm_words, ea.kpm_w32, p->g.csr_src, p->nnz,
                              p->kpm_csr, stream);
        if (st != PMA_OK)
            return fail(st, "mask packing failed: %s", hipGetErrorString(hipGetLastError()));
        ea.kpm_csr = p->kpm_csr;
    }
    // Automatic choices (measured on MI355X): the forward reads each query
    // row once, past the caches, so that its misses evict (and write back)
    // nothing (gene edge kernel 126 -> 112 us when the caches hold a previous
    // kernel's dirty lines, level when they hold clean ones; only a forward
    // repeated on the very same tokens loses, 96 -> 114 us); mixed and out
    // stores go past the caches in training (the backward reads them much
    // later; with the q loads, gene training step 0.870 -> 0.857 ms) and
    // where the workspace outgrows the 256 MB last-level cache; keep the
    // edge kernel's wavefronts resident and walking pieces when pieces are
    // short (then per-piece start-up latency dominates).
    const double ws_bytes = ((double)L + 2.0 * S_ws) * B * E * es;
    ea.nt = p->nt >= 0 ? p->nt : (save || ws_bytes > 256.0 * 1024 * 1024 ? 3 : 1);
    // (16 workgroups per CU: gene forward 151.8-152.5 -> 150.0-150.4 us cold
    // against 12, four alternations of 60 steps)
    ea.persist = p->persist >= 0 ? p->persist : (p->nnz < 32 * p->g.n_tasks ? 16 : 0);
    ea.fuse_out = fuse_out;
    ea.wo = o_w;
    ea.bo = o_b;
    ea.out = out;
    ea.fuse_in = fuse_in;
    ea.wq = q_w;
    ea.bq = q_b;
    ea.coop = p->coop;
    ea.max_pieces = p->g.max_degree > p->chunk ? (int)((p->g.max_degree + p->chunk - 1) / p->chunk) : 1;
    // Sample groups (wavefronts of 64 lanes over a target's B rows) and
    // XCDs: pinning each group to 8 / groups XCDs (where the group count
    // divides 8) gives each L2 the rows of one group only, which multiplies
    // its reuse by the group count. Running the groups one after another
    // instead keeps only one group's keys and values in flight, which pays
    // when all of them outgrow the 256 MB last-level cache and the L2 gain
    // is small: measured on MI355X, two groups over 350 MB (embed_dim 128,
    // B = 8, 100k sources) run 6% faster in turn, while 4 and 8 groups
    // (B = 32 at embed_dim 64; fp32 B = 16 at 128) are much faster pinned.
    const int64_t groups = (B * (E / (p->dtype == PMA_BF16 ? 8 : 4)) + 63) / 64;
    const bool in_turn = groups == 2 && ea.kv_bytes > ((uint64_t)256 << 20) && ea.persist == 0;
    ea.xcd_map = p->xcd_map >= 0 ? p->xcd_map : (in_turn ? 2 : 1);
    // Hot-row cache for the q-projecting kernel (no mask, no weights; opt-in):
    // each workgroup keeps the key/value rows of the most-read sources for
    // its sample group in LDS. Measured on MI355X it is slower on the
    // gene-regulatory workload (166 against 134 us per forward): the one
    // resident 16-wavefront workgroup per CU that the 128 KB cache needs runs
    // 4 wavefronts per SIMD instead of 7 and gives up the balancing of queued
    // workgroups, which costs more than the key/value reads it saves.
    if (fuse_in && p->hot && !kpm && !weights && ea.xcd_map == 1 && !no_alloc) {
        st = build_hot(p, ea.gather_src, S_ws, stream);
        if (st != PMA_OK)
            return fail(st, "hot-row index build failed");
        ea.hot_csr = p->hot_csr;
        ea.hot_src = p->hot_src;
        ea.n_hot = p->n_hot;
    }

    if (kpm && !pma::mask_supported(ea))
        return fail(PMA_E_UNSUPPORTED, "key_padding_mask with a workspace tensor of 2 GiB or more");

    // Steps 2-4 (and 5 when fused): scores, softmax and mix over the live edges.
    tm.begin(PMA_STAGE_EDGE);
    st = pma::launch_edge(ea, stream);
    tm.end();
    if (!save && !no_alloc) {
        p->probe_ea = ea;
        p->probe_ok = true;
    }
    if (st == PMA_OK && p->g.n_split > 0 && !pma::edge_merges_splits(ea)) {
        tm.begin(PMA_STAGE_MERGE);
        st = pma::launch_merge(ea, stream);
        tm.end();
    }
    if (st == PMA_OK && weights) {
        tm.begin(PMA_STAGE_WEIGHTS);
        st = pma::launch_weights(ea, stream);
        tm.end();
    }
    if (st != PMA_OK)
        return fail(st, "edge launch failed: %s", hipGetErrorString(hipGetLastError()));
    if (ea.fuse_out)
        return PMA_OK;   // out_proj ran in the edge and merge kernels

    // Step 5: join heads (already contiguous) and out_proj, back to (B, L, E),
    // visiting rows in mixed's storage order.
    tm.begin(PMA_STAGE_OUT);
    const pma::ProjOut oo{o_w, o_b, out, L * E, E};
    const int mixed_token_major = lay.m_b == E ? 1 : 0;
    pma::ProjArgs ao{mixed_ws, L * B, L, B, mixed_token_major, 1, {oo}};
    ao.x_token_major = mixed_token_major;
    ao.x3 = p->x3 && p->dtype == PMA_F32;
    st = pma::launch_proj(ao, E, p->dtype, stream);
    tm.end();
    if (st != PMA_OK)
        return fail(st, "out_proj launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

}  // namespace

PMA_API pma_status pma_forward(pma_plan *plan, int64_t batch, const void *query, const void *key,
                               const void *value, const void *q_w, const void *q_b,
                               const void *k_w, const void *k_b, const void *v_w,
                               const void *v_b, const void *o_w, const void *o_b, void *out,
                               float *weights, int average_attn_weights, hipStream_t stream)
{
    return forward_impl(plan, batch, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                        out, weights, average_attn_weights, nullptr, 0, nullptr, false, stream);
}

PMA_API pma_status pma_forward_static(pma_plan *plan, int64_t batch, const void *query,
                                      const void *key, const void *value, const void *q_w,
                                      const void *q_b, const void *k_w, const void *k_b,
                                      const void *v_w, const void *v_b, const void *o_w,
                                      const void *o_b, void *out, float *weights,
                                      int average_attn_weights, hipStream_t stream)
{
    return forward_impl(plan, batch, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                        out, weights, average_attn_weights, nullptr, 0, nullptr, true, stream);
}

PMA_API pma_status pma_forward_masked(pma_plan *plan, int64_t batch, const void *query,
                                      const void *key, const void *value, const void *q_w,
                                      const void *q_b, const void *k_w, const void *k_b,
                                      const void *v_w, const void *v_b, const void *o_w,
                                      const void *o_b, void *out, float *weights,
                                      int average_attn_weights, const uint8_t *key_padding_mask,
                                      int mask_per_sample, hipStream_t stream)
{
    g_err[0] = 0;
    if (!key_padding_mask)
        return fail(PMA_E_NULL, "key_padding_mask is NULL");
    if (mask_per_sample != 0 && mask_per_sample != 1)
        return fail(PMA_E_ARG, "mask_per_sample must be 0 or 1");
    return forward_impl(plan, batch, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                        out, weights, average_attn_weights, key_padding_mask, mask_per_sample,
                        nullptr, false, stream);
}

PMA_API pma_status pma_gather_probe(pma_plan *plan, hipStream_t stream)
{
    g_err[0] = 0;
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    if (!plan->probe_ok)
        return fail(PMA_E_ARG, "no inference forward on this plan's current workspace");
    const pma_status st = pma::launch_gather_probe(plan->probe_ea, stream);
    if (st == PMA_E_UNSUPPORTED)
        return fail(st, "the probe serves the 16-byte edge kernel with tensors under 2 GiB");
    if (st != PMA_OK)
        return fail(st, "probe launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

PMA_API pma_status pma_gather_ceiling(const void *table, uint64_t table_bytes, const int32_t *rows,
                                      int64_t n_rows, int64_t rows_per_wave, void *sink,
                                      hipStream_t stream)
{
    g_err[0] = 0;
    if (!table || !rows || !sink)
        return fail(PMA_E_NULL, "table, rows and sink must be device pointers");
    if (table_bytes < 1024 || table_bytes % 1024 != 0 || table_bytes >= ((uint64_t)1 << 32))
        return fail(PMA_E_ARG, "table_bytes must be a multiple of 1024 in [1024, 2^32)");
    if (n_rows < 1 || rows_per_wave < 1 || rows_per_wave > (1 << 20))
        return fail(PMA_E_ARG, "n_rows >= 1 and rows_per_wave in [1, 2^20] required");
    if ((n_rows + rows_per_wave - 1) / rows_per_wave > ((int64_t)1 << 30))
        return fail(PMA_E_ARG, "more than 2^30 wavefronts");
    const pma_status st = pma::launch_gather_ceiling(table, table_bytes, rows, n_rows, rows_per_wave,
                                                     sink, stream);
    if (st != PMA_OK)
        return fail(st, "gather ceiling launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

PMA_API size_t pma_train_bytes(const pma_plan *plan, int64_t batch)
{
    if (!plan || batch <= 0 || plan->E == 0)
        return 0;
    return save_layout(plan, batch).total;
}

PMA_API pma_status pma_forward_train(pma_plan *plan, int64_t batch, const void *query,
                                     const void *key, const void *value, const void *q_w,
                                     const void *q_b, const void *k_w, const void *k_b,
                                     const void *v_w, const void *v_b, const void *o_w,
                                     const void *o_b, void *out, float *weights,
                                     int average_attn_weights, const uint8_t *key_padding_mask,
                                     int mask_per_sample, void *save, hipStream_t stream)
{
    g_err[0] = 0;
    if (!save)
        return fail(PMA_E_NULL, "save is NULL");
    if (key_padding_mask && mask_per_sample != 0 && mask_per_sample != 1)
        return fail(PMA_E_ARG, "mask_per_sample must be 0 or 1");
    return forward_impl(plan, batch, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                        out, weights, average_attn_weights, key_padding_mask,
                        key_padding_mask ? mask_per_sample : 0, static_cast<char *>(save), false,
                        stream);
}

PMA_API pma_status pma_backward(pma_plan *plan, int64_t batch, const void *query,
                                const void *key, const void *value, const void *q_w,
                                const void *k_w, const void *v_w, const void *o_w, int has_bias,
                                const void *save, const void *grad_out,
                                const uint8_t *key_padding_mask, int mask_per_sample,
                                void *grad_query, void *grad_key, void *grad_value,
                                void *grad_q_w, void *grad_q_b, void *grad_k_w, void *grad_k_b,
                                void *grad_v_w, void *grad_v_b, void *grad_o_w, void *grad_o_b,
                                hipStream_t stream)
{
    g_err[0] = 0;
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    if (plan->E == 0)
        return fail(PMA_E_ARG, "the plan has no attention sizes (made by pma_create_graph)");
    if (batch <= 0)
        return fail(PMA_E_SIZE, "batch must be positive (got %lld)", (long long)batch);
    if (!query || !key || !value || !q_w || !k_w || !v_w || !o_w || !save || !grad_out ||
        !grad_query || !grad_key || !grad_value || !grad_q_w || !grad_k_w || !grad_v_w ||
        !grad_o_w)
        return fail(PMA_E_NULL, "a required pointer is NULL");
    if (has_bias != 0 && has_bias != 1)
        return fail(PMA_E_ARG, "has_bias must be 0 or 1");
    if (has_bias && (!grad_q_b || !grad_k_b || !grad_v_b || !grad_o_b))
        return fail(PMA_E_NULL, "a bias gradient pointer is NULL");
    if (key_padding_mask && mask_per_sample != 0 && mask_per_sample != 1)
        return fail(PMA_E_ARG, "mask_per_sample must be 0 or 1");
    pma_plan *p = plan;
    const int64_t B = batch, L = p->L, S = p->S, E = p->E, H = p->H, nnz = p->nnz;
    // a shared gradient output must belong to inputs of one shape
    if ((grad_key == grad_query || grad_value == grad_query) && L != S)
        return fail(PMA_E_ARG, "a key/value gradient shares the query's only when L == S");
    if (E / H > 64)
        return fail(PMA_E_UNSUPPORTED, "head size above 64 in the backward pass");
    if ((L > S ? L : S) * B * 2 * E > ((int64_t)1 << 40))
        return fail(PMA_E_UNSUPPORTED, "batch too large");
    // the per-position mask words are indexed with 32 bits
    if (key_padding_mask && (nnz + 4) * ((B + 31) / 32) >= ((int64_t)1 << 31))
        return fail(PMA_E_UNSUPPORTED, "key_padding_mask with nnz * ceil(batch / 32) of 2^31 or more");
    char err[256] = "";
    if (!p->g.csc_ptr) {
        pma_status st = pma::build_csc(&p->g, nnz, L, S, p->bchunk, p->bsub, stream, err, sizeof err);
        if (st != PMA_OK)
            return fail(st, "%s", err);
    }

    // scratch: dm, dq, dk, dv (plan dtype); for the 16-byte edge passes the
    // per-(target, sample, head) (m + log2 l, D), for the per-channel ones the
    // per-edge (p, dz) pairs; piece partials and weight-gradient partials (fp32)
    const pma_dtype dt = p->dtype;
    const size_t es = dt == PMA_BF16 ? 2 : 4;
    const int64_t RLr = B * L, RSr = B * S;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t b_dm = up(RLr * E * es), b_dkv = up(RSr * E * es);
    const SaveLayout sv0 = save_layout(p, B);
    const char *sb0 = static_cast<const char *>(save);
    const int64_t skv0 = train_compact(p) ? p->g.n_kv : S;   // saved key/value rows per sample
    const bool fast_edges =
        pma::bwd_edges_fast(E, H, dt, sb0 + sv0.q, sb0 + sv0.k,
                            sb0 + sv0.k + (size_t)B * skv0 * E * es, sb0 + sv0.mixed);
    const size_t b_pz = fast_edges ? up((size_t)L * B * H * 2 * 4)     // (m', D)
                                   : up((size_t)nnz * B * H * 2 * es); // (p, dz) pairs
    const size_t b_piece = up(pma::bwd_piece_scratch(p->g, B, E));
    const size_t b_wg = up(pma::wgrad_scratch(E, 4, RLr > RSr ? RLr : RSr));
    const size_t need = 2 * b_dm + 2 * b_dkv + b_pz + b_piece + b_wg;
    if (need > p->bw_bytes) {
        hipError_t e = hipStreamSynchronize(stream);
        if (p->bw)
            (void)hipFree(p->bw);
        p->bw = nullptr;
        p->bw_bytes = 0;
        if (e == hipSuccess)
            e = hipMalloc(&p->bw, need);
        if (e != hipSuccess)
            return fail(e == hipErrorOutOfMemory ? PMA_E_OOM : PMA_E_DEVICE,
                        "backward scratch of %zu bytes: %s", need, hipGetErrorString(e));
        p->bw_bytes = need;
    }
    char *cur = p->bw;
    auto take = [&](size_t n) {
        char *r = cur;
        cur += n;
        return r;
    };
    void *dm = take(b_dm), *dq = take(b_dm), *dk = take(b_dkv), *dv = take(b_dkv);
    void *PZ = take(b_pz);
    float *part = reinterpret_cast<float *>(take(b_piece));
    float *wpart = reinterpret_cast<float *>(take(b_wg));

    const SaveLayout sv = save_layout(p, B);
    const char *sb = static_cast<const char *>(save);
    pma_status st = PMA_OK;
    auto ok = [&](pma_status x) {
        if (st == PMA_OK)
            st = x;
    };

    // out_proj: dm = dO Wo
    {
        pma::RowMM r{{grad_out}, {o_w}, 1, dm, RLr, 0};
        ok(pma::launch_rowmm(r, E, dt, stream));
    }

    // scores, softmax and mix
    pma::BwdArgs a;
    a.B = (int)B;
    a.L = (int)L;
    a.S = (int)S;
    a.E = (int)E;
    a.H = (int)H;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)(E / H)));
    a.inv_sqrt_d = (float)(1.0 / sqrt((double)(E / H)));
    // keys and values as the training forward saved them: n_kv rows per
    // sample (read sources only) or all S
    const bool compact = train_compact(p);
    a.Skv = (int)(compact ? p->g.n_kv : S);
    a.kv_src = compact ? p->g.csr_kv : p->g.csr_src;
    a.q = sb + sv.q;
    a.k = sb + sv.k;
    a.v = sb + sv.k + (size_t)B * a.Skv * E * es;
    a.mixed = sb + sv.mixed;
    a.ml = reinterpret_cast<const float *>(sb + sv.ml);
    a.dm = dm;
    const pma::GraphDev &gd = p->g;
    a.row_ptr = gd.row_ptr;
    a.csr_src = gd.csr_src;
    a.csc_ptr = gd.csc_ptr;
    a.csc_tgt = gd.csc_tgt;
    a.csc_pos = gd.csc_pos;
    a.t_target = gd.task_target;
    a.t_begin = gd.task_begin;
    a.t_end = gd.task_end;
    a.t_slot = gd.task_slot;
    a.ts_target = gd.split_target;
    a.ts_slot0 = gd.split_slot0;
    a.ts_count = gd.split_count;
    a.s_source = gd.s_source;
    a.s_begin = gd.s_begin;
    a.s_end = gd.s_end;
    a.s_slot = gd.s_slot;
    a.ss_source = gd.ss_source;
    a.ss_slot0 = gd.ss_slot0;
    a.ss_count = gd.ss_count;
    a.n_ttasks = gd.n_tasks;
    a.n_tsplit = gd.n_split;
    a.n_stasks = gd.n_stasks;
    a.n_ssplit = gd.n_ssplit;
    a.n_tslots = gd.n_slots;
    a.n_sslots = gd.n_sslots;
    for (int k = 0; k <= pma::kBands; ++k)
        a.s_band_off[k] = gd.s_band_off[k];
    a.banded = gd.s_banded ? 1 : 0;
    a.t_order = p->border;
    a.s_order = p->bsorder;
    a.t_pf = p->bpf;
    a.nt = p->bnt;
    a.kpm_bits = nullptr;
    a.kpm_words = 0;
    a.kpm_csr = nullptr;
    a.kpm_w32 = 0;
    if (key_padding_mask) {
        pma_status st2 = ensure_workspace(p, B, false, stream);
        if (st2 != PMA_OK)
            return st2;
        ok(pma::pack_mask(key_padding_mask, mask_per_sample ? S : 0, B, S, p->kpm_bits, stream));
        a.kpm_bits = p->kpm_bits;
        a.kpm_words = (int)((B + 63) / 64);
        a.kpm_w32 = (int)((B + 31) / 32);
        ok(pma::gather_mask(p->kpm_bits, a.kpm_words, a.kpm_w32, gd.csr_src, p->nnz, p->kpm_csr,
                            stream));
        a.kpm_csr = p->kpm_csr;
    }
    a.PZ = fast_edges ? nullptr : PZ;
    a.mD = fast_edges ? static_cast<float *>(PZ) : nullptr;
    a.part_q = part;
    a.part_kv = part + (size_t)gd.n_slots * B * E;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    ok(pma::launch_bwd_edges(a, dt, stream));

    // weight and bias gradients of the four maps
    {
        pma::WGrad w;
        w.np = 4;
        w.E = (int)E;
        w.nwg = 0;
        w.part = wpart;
        w.p[0] = {grad_out, sb + sv.mixed, RLr, grad_o_w, has_bias ? grad_o_b : nullptr};
        w.p[1] = {dq, query, RLr, grad_q_w, has_bias ? grad_q_b : nullptr};
        w.p[2] = {dk, key, RSr, grad_k_w, has_bias ? grad_k_b : nullptr};
        w.p[3] = {dv, value, RSr, grad_v_w, has_bias ? grad_v_b : nullptr};
        if (compact && RSr < ((int64_t)1 << 31)) {
            // dk and dv are zero on the sources no edge reads: only the
            // read sources' rows of dk, dv and the key / value tokens
            for (int i = 2; i < 4; ++i) {
                w.p[i].rows = B * gd.n_kv;
                w.p[i].list = gd.kv_rows;
                w.p[i].n = gd.n_kv;
                w.p[i].n_in = S;
            }
        }
        ok(pma::launch_wgrad(w, dt, stream));
    }

    // token gradients dX = dY W, summed over the maps that read one tensor
    const void *G[3] = {dq, dk, dv};
    const void *Wm[3] = {q_w, k_w, v_w};
    void *outs[3] = {grad_query, grad_key, grad_value};
    const int64_t rows[3] = {RLr, RSr, RSr};
    for (int i = 0; i < 3; ++i) {
        int j = 0;
        while (j < i && outs[j] != outs[i])
            ++j;
        if (j < i)
            continue;   // handled with its first use
        pma::RowMM r{{}, {}, 0, outs[i], rows[i], 0};
        for (int k = i; k < 3; ++k) {
            if (outs[k] == outs[i]) {
                r.x[r.nin] = G[k];
                r.w[r.nin] = Wm[k];
                ++r.nin;
            }
        }
        ok(pma::launch_rowmm(r, E, dt, stream));
    }
    if (st != PMA_OK)
        return fail(st, "backward launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

namespace {

// Checks shared by the PackedLinear calls; grows the plan's scratch to hold
// fp32 partials of `slots` rows and `nbuf` node-major copies of up to
// max(L, S) rows, all of R = batch * channels values.
pma_status linear_common(pma_plan *p, int64_t batch, int64_t channels, int64_t slots, int nbuf,
                         char **ws)
{
    if (!p)
        return fail(PMA_E_NULL, "plan is NULL");
    if (batch <= 0 || channels <= 0)
        return fail(PMA_E_SIZE, "batch and channels must be positive (got %lld, %lld)",
                    (long long)batch, (long long)channels);
    const int64_t R = batch * channels;
    const int64_t rows = (p->L > p->S ? p->L : p->S);
    if (R > kI32 || rows * R > ((int64_t)1 << 40))
        return fail(PMA_E_UNSUPPORTED, "batch * channels too large");
    const size_t es = p->dtype == PMA_BF16 ? 2 : 4;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t need = up((size_t)(slots > 0 ? slots : 1) * R * sizeof(float)) +
                        (size_t)nbuf * up((size_t)rows * R * es);
    if (need > p->lin_bytes) {
        if (p->lin) {
            (void)hipDeviceSynchronize();
            (void)hipFree(p->lin);
        }
        p->lin = nullptr;
        p->lin_bytes = 0;
        hipError_t e = hipMalloc(&p->lin, need);
        if (e != hipSuccess)
            return fail(e == hipErrorOutOfMemory ? PMA_E_OOM : PMA_E_DEVICE,
                        "PackedLinear scratch of %zu bytes: %s", need, hipGetErrorString(e));
        p->lin_bytes = need;
    }
    *ws = p->lin;
    return PMA_OK;
}

}  // namespace

PMA_API pma_status pma_linear_forward(pma_plan *plan, int64_t batch, int64_t channels,
                                      const void *x, const void *weight, const void *bias,
                                      void *out, hipStream_t stream)
{
    g_err[0] = 0;
    if (plan && (!x || !weight || !out))
        return fail(PMA_E_NULL, "x, weight or out is NULL");
    const pma_dtype dt = plan ? plan->dtype : PMA_F32;
    const void *user[2] = {x, out};
    // Read the batch-first tensors directly when a sample's channels fill
    // 16-byte chunks (or there is one sample); else go node-major.
    const bool direct = batch == 1 || pma::lin_vec(channels, dt, user, 2) > 1;
    char *ws = nullptr;
    pma_status st = linear_common(plan, batch, channels, plan ? plan->g.n_slots : 0,
                                  direct ? 0 : 2, &ws);
    if (st != PMA_OK)
        return st;
    const pma::GraphDev &g = plan->g;
    const int64_t R = batch * channels, L = plan->L, S = plan->S;
    const size_t es = dt == PMA_BF16 ? 2 : 4;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t b_part = up((size_t)(g.n_slots > 0 ? g.n_slots : 1) * R * sizeof(float));
    const size_t b_row = up((size_t)(L > S ? L : S) * R * es);
    pma::LinArgs a;
    a.R = (int)R;
    if (direct) {
        a.x = x;
        a.y = out;
        a.Cs = (int)channels;
        a.sn_in = channels;
        a.sb_in = S * channels;
        a.sn_out = channels;
        a.sb_out = L * channels;
    } else {
        a.x = ws + b_part;
        a.y = ws + b_part + b_row;
        a.Cs = (int)R;
        a.sn_in = a.sn_out = R;
        a.sb_in = a.sb_out = 0;
        st = pma::launch_transpose(x, const_cast<void *>(a.x), batch, S, channels, dt, stream);
    }
    a.w = weight;
    a.bias = bias;
    a.idx = g.csr_src;
    a.eid = g.csr_eid;
    a.t_row = g.task_target;
    a.t_begin = g.task_begin;
    a.t_end = g.task_end;
    a.t_slot = g.task_slot;
    a.n_tasks = g.n_tasks;
    a.s_row = g.split_target;
    a.s_slot0 = g.split_slot0;
    a.s_count = g.split_count;
    a.n_split = g.n_split;
    a.part = reinterpret_cast<float *>(ws);
    const void *ptrs[2] = {a.x, a.y};
    if (st == PMA_OK)
        st = pma::launch_spmm(a, dt, pma::lin_vec(a.Cs, dt, ptrs, 2), stream);
    if (st == PMA_OK && !direct)
        st = pma::launch_transpose(a.y, out, L, batch, channels, dt, stream);
    if (st != PMA_OK)
        return fail(st, "PackedLinear launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

PMA_API pma_status pma_linear_backward(pma_plan *plan, int64_t batch, int64_t channels,
                                       const void *x, const void *weight, const void *grad_out,
                                       void *grad_x, void *grad_weight, void *grad_bias,
                                       hipStream_t stream)
{
    g_err[0] = 0;
    if (plan && (!x || !weight || !grad_out || !grad_x || !grad_weight))
        return fail(PMA_E_NULL, "a required pointer is NULL");
    if (plan && (batch <= 0 || channels <= 0))
        return fail(PMA_E_SIZE, "batch and channels must be positive (got %lld, %lld)",
                    (long long)batch, (long long)channels);
    if (plan && !plan->g.csc_ptr) {
        char err[256] = "";
        pma_status st = pma::build_csc(&plan->g, plan->nnz, plan->L, plan->S, plan->bchunk, plan->bsub, stream, err,
                                       sizeof err);
        if (st != PMA_OK)
            return fail(st, "%s", err);
    }
    const pma_dtype dt = plan ? plan->dtype : PMA_F32;
    const void *user[3] = {x, grad_out, grad_x};
    const bool direct = batch == 1 || pma::lin_vec(channels, dt, user, 3) > 1;
    char *ws = nullptr;
    pma_status st = linear_common(plan, batch, channels, plan ? plan->g.n_sslots : 0,
                                  direct ? 0 : 3, &ws);
    if (st != PMA_OK)
        return st;
    const pma::GraphDev &g = plan->g;
    const int64_t R = batch * channels, L = plan->L, S = plan->S;
    const size_t es = dt == PMA_BF16 ? 2 : 4;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t b_part = up((size_t)(g.n_sslots > 0 ? g.n_sslots : 1) * R * sizeof(float));
    const size_t b_row = up((size_t)(L > S ? L : S) * R * es);
    // rows of x, dy and dx: batch-first segments of C, or node-major rows
    const void *xr = x, *gr = grad_out;
    void *dxr = grad_x;
    int Cs = (int)channels;
    int64_t snx = channels, sbx = S * channels, sng = channels, sbg = L * channels;
    if (!direct) {
        xr = ws + b_part;
        gr = ws + b_part + b_row;
        dxr = ws + b_part + 2 * b_row;
        Cs = (int)R;
        snx = sng = R;
        sbx = sbg = 0;
        st = pma::launch_transpose(x, const_cast<void *>(xr), batch, S, channels, dt, stream);
        if (st == PMA_OK)
            st = pma::launch_transpose(grad_out, const_cast<void *>(gr), batch, L, channels, dt,
                                       stream);
    }
    // input gradient: the same product over the source-major pieces
    pma::LinArgs a;
    a.R = (int)R;
    a.Cs = Cs;
    a.sn_in = sng;
    a.sb_in = sbg;
    a.sn_out = snx;
    a.sb_out = sbx;
    a.x = gr;
    a.w = weight;
    a.bias = nullptr;
    a.y = dxr;
    a.idx = g.csc_tgt;
    a.eid = g.csc_eid;
    a.t_row = g.s_source;
    a.t_begin = g.s_begin;
    a.t_end = g.s_end;
    a.t_slot = g.s_slot;
    a.n_tasks = g.n_stasks;
    a.s_row = g.ss_source;
    a.s_slot0 = g.ss_slot0;
    a.s_count = g.ss_count;
    a.n_split = g.n_ssplit;
    a.part = reinterpret_cast<float *>(ws);
    const void *ptrs[3] = {xr, gr, dxr};
    const int vec = pma::lin_vec(Cs, dt, ptrs, 3);
    if (st == PMA_OK)
        st = pma::launch_spmm(a, dt, vec, stream);
    if (st == PMA_OK && !direct)
        st = pma::launch_transpose(dxr, grad_x, S, batch, channels, dt, stream);
    if (st == PMA_OK) {
        pma::RowDots d;
        d.csr_src = g.csr_src;
        d.csr_tgt = g.csr_tgt;
        d.csr_eid = g.csr_eid;
        d.nnz = plan->nnz;
        d.L = L;
        d.R = (int)R;
        d.Cs = Cs;
        d.snx = snx;
        d.sbx = sbx;
        d.sng = sng;
        d.sbg = sbg;
        d.x = xr;
        d.dy = gr;
        d.dw = grad_weight;
        d.db = grad_bias;
        st = pma::launch_lin_rowdots(d, dt, vec, stream);
    }
    if (st != PMA_OK)
        return fail(st, "PackedLinear backward launch failed: %s",
                    hipGetErrorString(hipGetLastError()));
    return PMA_OK;
}

PMA_API pma_status pma_profile(pma_plan *plan, int enable)
{
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    if (enable != 0 && enable != 1)
        return fail(PMA_E_ARG, "enable must be 0 or 1");
    plan->prof = enable ? (1u << PMA_NUM_STAGES) - 1u : 0u;
    return PMA_OK;
}

PMA_API pma_status pma_profile_stages(pma_plan *plan, unsigned mask)
{
    if (!plan)
        return fail(PMA_E_NULL, "plan is NULL");
    if (mask >> PMA_NUM_STAGES)
        return fail(PMA_E_ARG, "mask has bits beyond the %d stages", (int)PMA_NUM_STAGES);
    plan->prof = mask;
    return PMA_OK;
}

PMA_API pma_status pma_profile_read(pma_plan *plan, double *ms, int64_t *calls)
{
    if (!plan || !ms || !calls)
        return fail(PMA_E_NULL, "NULL argument");
    pma_status st = PMA_OK;
    for (auto &ev : plan->pending) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(ev.b);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&t, ev.a, ev.b);
        if (e != hipSuccess)
            st = fail(PMA_E_DEVICE, "event timing: %s", hipGetErrorString(e));
        else {
            plan->ms[ev.stage] += t;
            plan->calls[ev.stage] += 1;
        }
        plan->pool.push_back(ev.a);
        plan->pool.push_back(ev.b);
    }
    plan->pending.clear();
    for (int i = 0; i < PMA_NUM_STAGES; ++i) {
        ms[i] = plan->ms[i];
        calls[i] = plan->calls[i];
        plan->ms[i] = 0;
        plan->calls[i] = 0;
    }
    return st;
}
