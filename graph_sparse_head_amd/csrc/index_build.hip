// Device-side index build: edges grouped by target with sources ascending
// (CSR by target), duplicate-pair detection, and the split of every target
// into pieces of at most `chunk` edges.
//
// The softmax of the kpnn2 PackedMultiheadAttention page runs over "the edges
// into each target" ("Notes", step 3); grouping the edges by target makes
// each softmax one contiguous segment. Sorting each segment by source makes
// the layout unique (pairs do not repeat), so the build is deterministic, and
// puts a repeated pair next to its twin, which is how the constructor's
// "must not repeat a (source, target) pair" rule is checked.
//
// Sorting is a stable least-significant-digit radix sort on 8-bit digits:
// source digits first, then target digits. Each pass counts digits per tile,
// scans the (digit, tile) counts, and scatters every tile in order, so equal
// digits keep their relative order without atomics.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "pma_internal.h"

namespace pma {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kTile = kThreads * kItems;  // 2048 elements per tile
// Pieces run longest first in buckets of 16 edges, and by ascending target
// inside a bucket, so that wavefronts resident together touch nearby token
// rows (fewer address-translation misses than a strict length order).
constexpr int kLenBucketShift = 4;

#define PMA_TRY(call)                                                                  \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            snprintf(err, errlen, "%s failed: %s", #call, hipGetErrorString(e_));      \
            st = (e_ == hipErrorOutOfMemory) ? PMA_E_OOM : PMA_E_DEVICE;               \
            goto fail;                                                                 \
        }                                                                              \
    } while (0)

// Exclusive prefix sum of one value per thread over a 256-thread block.
__device__ int block_exclusive_scan(int v, int *lds, int *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        lds[wid] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        int s = lds[w];
        before += (w < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// ---- device-wide exclusive scan ------------------------------------------

__global__ void __launch_bounds__(kThreads) scan_tile_sums(const int32_t *in, int64_t n,
                                                           int32_t *tile_sums)
{
    __shared__ int lds[kThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
    int s = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j)
        s += (base + j < n) ? in[base + j] : 0;
    int tot;
    block_exclusive_scan(s, lds, &tot);
    if (threadIdx.x == 0)
        tile_sums[blockIdx.x] = tot;
}

// One block scans all tile sums in place (exclusive), carrying across rounds.
__global__ void __launch_bounds__(kThreads) scan_tile_offsets(int32_t *tile_sums, int64_t nt,
                                                              int32_t *total)
{
    __shared__ int lds[kThreads / 64];
    int carry = 0;
    for (int64_t base = 0; base < nt; base += kThreads) {
        int64_t i = base + threadIdx.x;
        int v = (i < nt) ? tile_sums[i] : 0;
        int tot;
        int ex = block_exclusive_scan(v, lds, &tot);
        if (i < nt)
            tile_sums[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0 && total)
        *total = carry;
}

__global__ void __launch_bounds__(kThreads) scan_apply(const int32_t *in, int32_t *out,
                                                       int64_t n, const int32_t *tile_offs)
{
    __shared__ int lds[kThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
    int v[kItems];
    int s = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        v[j] = (base + j < n) ? in[base + j] : 0;
        s += v[j];
    }
    int tot;
    int run = tile_offs[blockIdx.x] + block_exclusive_scan(s, lds, &tot);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        if (base + j < n)
            out[base + j] = run;
        run += v[j];
    }
}

// ---- radix sort pass -------------------------------------------------------

__global__ void __launch_bounds__(kThreads) radix_count(const int32_t *keys, const int32_t *perm,
                                                        int64_t n, int shift, int32_t *counts,
                                                        int64_t ntiles)
{
    __shared__ int hist[256];
    hist[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTile;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        int64_t i = base + j * kThreads + threadIdx.x;
        if (i < n)
            atomicAdd(&hist[(keys[perm[i]] >> shift) & 255], 1);
    }
    __syncthreads();
    counts[(int64_t)threadIdx.x * ntiles + blockIdx.x] = hist[threadIdx.x];
}

// Thread `d` walks the tile in order and moves the elements of digit d to
// their scanned offsets: a stable scatter without atomics.
__global__ void __launch_bounds__(kThreads) radix_scatter(const int32_t *keys,
                                                          const int32_t *perm_in, int64_t n,
                                                          int shift, const int32_t *offs,
                                                          int64_t ntiles, int32_t *perm_out)
{
    __shared__ int32_t val[kTile];
    __shared__ uint32_t dig4[kTile / 4];
    uint8_t *dig = reinterpret_cast<uint8_t *>(dig4);
    const int64_t base = (int64_t)blockIdx.x * kTile;
    const int cnt = (int)((n - base) < kTile ? (n - base) : kTile);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        int i = j * kThreads + threadIdx.x;
        if (i < cnt) {
            int32_t v = perm_in[base + i];
            val[i] = v;
            dig[i] = (uint8_t)((keys[v] >> shift) & 255);
        } else {
            dig[i] = 0;
        }
    }
    __syncthreads();
    const uint32_t me = threadIdx.x;
    int64_t pos = offs[(int64_t)me * ntiles + blockIdx.x];
    const int words = (cnt + 3) >> 2;
    for (int w = 0; w < words; ++w) {
        uint32_t d4 = dig4[w];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int i = w * 4 + k;
            if (((d4 >> (8 * k)) & 255) == me && i < cnt)
                perm_out[pos++] = val[i];
        }
    }
}

__global__ void iota_kernel(int32_t *a, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        a[i] = (int32_t)i;
}

// Row pointers of a sorted edge list: ptr[k] = the first position j whose key
// is at least k, for k = 0 .. K, with key(j) = key[perm[j]] (or key[j] when
// perm is null) ascending in j. One thread per k, by binary search: counting
// degrees with atomics serialises on the few nodes that hold a large share of
// the edges (a Zipf-popular source feeds a fifth of them).
__global__ void bounds_kernel(const int32_t *key, const int32_t *perm, int64_t n, int64_t K,
                              int32_t *ptr)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k > K)
        return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (key[perm ? perm[mid] : mid] >= k)
            hi = mid;
        else
            lo = mid + 1;
    }
    ptr[k] = (int32_t)lo;
}

// CSR arrays from the sorted permutation, and the duplicate check: after the
// sort a repeated (source, target) pair sits next to its twin.
__global__ void csr_fill(const int32_t *perm, const int32_t *src, const int32_t *tgt, int64_t nnz,
                         int32_t *csr_src, int32_t *csr_tgt, int32_t *csr_eid, int32_t *dup)
{
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= nnz)
        return;
    int32_t e = perm[p];
    int32_t s = src[e], t = tgt[e];
    csr_src[p] = s;
    csr_tgt[p] = t;
    csr_eid[p] = e;
    if (p > 0) {
        int32_t e0 = perm[p - 1];
        if (src[e0] == s && tgt[e0] == t)
            *dup = 1;
    }
}

// Sources that some edge reads (used[s] = 1), their compact numbering and
// the edges' sources in that numbering (the key/value workspace then holds
// only rows that are read).
__global__ void mark_used(const int32_t *csr_src, int64_t nnz, int32_t *used)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p < nnz)
        used[csr_src[p]] = 1;   // every writer stores the same value
}

__global__ void kv_rows_fill(const int32_t *used, const int32_t *kv_map, int64_t S, int32_t *kv_rows)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s < S && used[s])
        kv_rows[kv_map[s]] = (int32_t)s;
}

__global__ void kv_remap(const int32_t *csr_src, const int32_t *kv_map, int64_t nnz, int32_t *csr_kv)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p < nnz)
        csr_kv[p] = kv_map[csr_src[p]];
}

// Per target: number of pieces, partial slots and split flag.
__global__ void split_count_kernel(const int32_t *row_ptr, int64_t L, int chunk, int32_t *n_piece,
                                   int32_t *n_slot, int32_t *is_split, int32_t *max_deg)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= L)
        return;
    int32_t g = row_ptr[t + 1] - row_ptr[t];
    int32_t n = g > chunk ? (int32_t)((g + (int64_t)chunk - 1) / chunk) : 1;
    n_piece[t] = n;
    n_slot[t] = n > 1 ? n : 0;
    is_split[t] = n > 1 ? 1 : 0;
    atomicMax(max_deg, g);
}

__global__ void split_fill_kernel(const int32_t *row_ptr, int64_t L, int chunk,
                                  const int32_t *piece_base, const int32_t *slot_base,
                                  const int32_t *split_base, int32_t *t_target, int32_t *t_begin,
                                  int32_t *t_end, int32_t *t_slot, int32_t *t_split, int32_t *t_key,
                                  int32_t *s_target, int32_t *s_slot0, int32_t *s_count)
{
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= L)
        return;
    const int64_t r0 = row_ptr[t], g = row_ptr[t + 1] - r0;
    const int64_t n = g > chunk ? (g + chunk - 1) / chunk : 1;
    const int64_t pb = piece_base[t];
    for (int64_t j = 0; j < n; ++j) {
        int64_t b = r0 + (j * g) / n, e = r0 + ((j + 1) * g) / n;
        t_target[pb + j] = (int32_t)t;
        t_begin[pb + j] = (int32_t)b;
        t_end[pb + j] = (int32_t)e;
        t_slot[pb + j] = n > 1 ? (int32_t)(slot_base[t] + j) : -1;
        t_split[pb + j] = n > 1 ? split_base[t] : -1;
        t_key[pb + j] = (chunk - (int32_t)(e - b)) >> kLenBucketShift;  // longest buckets first
    }
    if (n > 1) {
        const int32_t k = split_base[t];
        s_target[k] = (int32_t)t;
        s_slot0[k] = slot_base[t];
        s_count[k] = (int32_t)n;
    }
}

__global__ void gather5_kernel(const int32_t *perm, int64_t n, const int32_t *a0,
                               const int32_t *a1, const int32_t *a2, const int32_t *a3,
                               const int32_t *a4, int32_t *o0, int32_t *o1, int32_t *o2,
                               int32_t *o3, int32_t *o4)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    int32_t p = perm[i];
    o0[i] = a0[p];
    o1[i] = a1[p];
    o2[i] = a2[p];
    o3[i] = a3[p];
    o4[i] = a4[p];
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

// Exclusive scan of n values (in -> out, may alias); writes the total to
// *total_dev if not null. tmp holds ceil(n / kTile) ints.
hipError_t scan_exclusive(const int32_t *in, int32_t *out, int64_t n, int32_t *total_dev,
                          int32_t *tmp, hipStream_t s)
{
    if (n <= 0) {
        if (total_dev)
            return hipMemsetAsync(total_dev, 0, sizeof(int32_t), s);
        return hipSuccess;
    }
    const int64_t nt = (n + kTile - 1) / kTile;
    scan_tile_sums<<<(unsigned)nt, kThreads, 0, s>>>(in, n, tmp);
    scan_tile_offsets<<<1, kThreads, 0, s>>>(tmp, nt, total_dev);
    scan_apply<<<(unsigned)nt, kThreads, 0, s>>>(in, out, n, tmp);
    return hipGetLastError();
}

int bits_for(int64_t maxval)
{
    int b = 0;
    while (b < 63 && (int64_t(1) << b) <= maxval)
        ++b;
    return b;
}

// Stable sort of `perm` (n entries) by keys[perm[i]] over `bits` low bits.
// Uses perm_tmp (n), counts (256 * tiles) and scan_tmp (>= 256 * tiles / kTile + 1).
hipError_t radix_sort_perm(const int32_t *keys, int bits, int32_t *&perm, int32_t *&perm_tmp,
                           int64_t n, int32_t *counts, int32_t *scan_tmp, hipStream_t s)
{
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int shift = 0; shift < bits; shift += 8) {
        radix_count<<<(unsigned)ntiles, kThreads, 0, s>>>(keys, perm, n, shift, counts, ntiles);
        hipError_t e = scan_exclusive(counts, counts, 256 * ntiles, nullptr, scan_tmp, s);
        if (e != hipSuccess)
            return e;
        radix_scatter<<<(unsigned)ntiles, kThreads, 0, s>>>(keys, perm, n, shift, counts, ntiles,
                                                            perm_tmp);
        int32_t *t = perm;
        perm = perm_tmp;
        perm_tmp = t;
    }
    return hipGetLastError();
}

}  // namespace

void free_graph(GraphDev *g)
{
    int32_t **ptrs[] = {&g->row_ptr,     &g->csr_src,     &g->csr_tgt,    &g->csr_eid,
                        &g->task_target, &g->task_begin,  &g->task_end,   &g->task_slot,
                        &g->task_split,  &g->split_target, &g->split_slot0, &g->split_count,
                        &g->csr_kv,      &g->kv_rows,     &g->csc_ptr,    &g->csc_tgt,
                        &g->csc_pos,     &g->csc_eid,     &g->s_source,   &g->s_begin,    &g->s_end,
                        &g->s_slot,      &g->ss_source,   &g->ss_slot0,   &g->ss_count};
    for (int32_t **p : ptrs) {
        if (*p)
            (void)hipFree(*p);
        *p = nullptr;
    }
}

pma_status build_graph(const int32_t *h_src, const int32_t *h_tgt, int64_t nnz, int64_t L,
                       int64_t S, int chunk, hipStream_t stream, GraphDev *g, char *err,
                       size_t errlen)
{
    pma_status st = PMA_OK;
    int32_t *d_src = nullptr, *d_tgt = nullptr, *perm = nullptr, *perm_tmp = nullptr;
    int32_t *counts = nullptr, *scan_tmp = nullptr, *small = nullptr;
    int32_t *n_piece = nullptr, *n_slot = nullptr, *is_split = nullptr;
    int32_t *piece_base = nullptr, *slot_base = nullptr, *split_base = nullptr;
    int32_t *t_target = nullptr, *t_begin = nullptr, *t_end = nullptr, *t_slot = nullptr,
            *t_split = nullptr, *t_key = nullptr, *tperm = nullptr, *tperm_tmp = nullptr;
    int32_t *used = nullptr, *kv_map = nullptr;
    int32_t h_small[8] = {0};
    // longest array any scan below sees
    const int64_t n_sort = std::max(std::max(nnz, L), S);
    const int64_t ntiles = (n_sort + kTile - 1) / kTile;
    const int64_t count_len = 256 * ntiles;
    const int64_t scan_len = (count_len > n_sort ? count_len : n_sort) / kTile + 2;
    const size_t i4 = sizeof(int32_t);

    // small[]: 0 dup flag, 1 n_tasks, 2 n_slots, 3 n_split, 4 max degree,
    // 5 distinct sources read
    PMA_TRY(hipMalloc(&d_src, nnz * i4));
    PMA_TRY(hipMalloc(&d_tgt, nnz * i4));
    PMA_TRY(hipMalloc(&perm, nnz * i4));
    PMA_TRY(hipMalloc(&perm_tmp, nnz * i4));
    PMA_TRY(hipMalloc(&counts, count_len * i4));
    PMA_TRY(hipMalloc(&scan_tmp, scan_len * i4));
    PMA_TRY(hipMalloc(&small, 8 * i4));
    PMA_TRY(hipMalloc(&g->row_ptr, (L + 1) * i4));
    // csr_src carries kSrcPad zero entries past nnz so that kernels may read a
    // fixed number of indices at a time without clamping.
    PMA_TRY(hipMalloc(&g->csr_src, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMemsetAsync(g->csr_src + nnz, 0, kSrcPad * i4, stream));
    PMA_TRY(hipMalloc(&g->csr_tgt, nnz * i4));
    PMA_TRY(hipMalloc(&g->csr_eid, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMemsetAsync(g->csr_eid + nnz, 0, kSrcPad * i4, stream));
    PMA_TRY(hipMalloc(&n_piece, L * i4));
    PMA_TRY(hipMalloc(&n_slot, L * i4));
    PMA_TRY(hipMalloc(&is_split, L * i4));
    PMA_TRY(hipMalloc(&piece_base, L * i4));
    PMA_TRY(hipMalloc(&slot_base, L * i4));
    PMA_TRY(hipMalloc(&split_base, L * i4));
    PMA_TRY(hipMalloc(&used, S * i4));
    PMA_TRY(hipMalloc(&kv_map, S * i4));
    PMA_TRY(hipMalloc(&g->kv_rows, S * i4));
    PMA_TRY(hipMalloc(&g->csr_kv, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMemsetAsync(g->csr_kv + nnz, 0, kSrcPad * i4, stream));
    PMA_TRY(hipMemsetAsync(used, 0, S * i4, stream));

    PMA_TRY(hipMemcpyAsync(d_src, h_src, nnz * i4, hipMemcpyHostToDevice, stream));
    PMA_TRY(hipMemcpyAsync(d_tgt, h_tgt, nnz * i4, hipMemcpyHostToDevice, stream));
    PMA_TRY(hipMemsetAsync(small, 0, 8 * i4, stream));

    // 1. sort edge ids by (target, source)
    iota_kernel<<<grid_for(nnz, 256), 256, 0, stream>>>(perm, nnz);
    PMA_TRY(radix_sort_perm(d_src, bits_for(S - 1), perm, perm_tmp, nnz, counts, scan_tmp, stream));
    PMA_TRY(radix_sort_perm(d_tgt, bits_for(L - 1), perm, perm_tmp, nnz, counts, scan_tmp, stream));
    csr_fill<<<grid_for(nnz, 256), 256, 0, stream>>>(perm, d_src, d_tgt, nnz, g->csr_src,
                                                     g->csr_tgt, g->csr_eid, small + 0);
    // 1b. compact numbering of the sources that are read
    mark_used<<<grid_for(nnz, 256), 256, 0, stream>>>(g->csr_src, nnz, used);
    PMA_TRY(scan_exclusive(used, kv_map, S, small + 5, scan_tmp, stream));
    kv_rows_fill<<<grid_for(S, 256), 256, 0, stream>>>(used, kv_map, S, g->kv_rows);
    kv_remap<<<grid_for(nnz, 256), 256, 0, stream>>>(g->csr_src, kv_map, nnz, g->csr_kv);
    // 2. row pointers
    bounds_kernel<<<grid_for(L + 1, 256), 256, 0, stream>>>(g->csr_tgt, nullptr, nnz, L, g->row_ptr);
    // 3. pieces per target
    split_count_kernel<<<grid_for(L, 256), 256, 0, stream>>>(g->row_ptr, L, chunk, n_piece, n_slot,
                                                             is_split, small + 4);
    PMA_TRY(scan_exclusive(n_piece, piece_base, L, small + 1, scan_tmp, stream));
    PMA_TRY(scan_exclusive(n_slot, slot_base, L, small + 2, scan_tmp, stream));
    PMA_TRY(scan_exclusive(is_split, split_base, L, small + 3, scan_tmp, stream));
    PMA_TRY(hipGetLastError());
    PMA_TRY(hipMemcpyAsync(h_small, small, 8 * i4, hipMemcpyDeviceToHost, stream));
    PMA_TRY(hipStreamSynchronize(stream));
    if (h_small[0]) {
        snprintf(err, errlen, "target_index/source_index repeat a (source, target) pair");
        st = PMA_E_INDEX_DUPLICATE;
        goto fail;
    }
    g->n_tasks = h_small[1];
    g->n_slots = h_small[2];
    g->n_split = h_small[3];
    g->max_degree = h_small[4];
    g->n_kv = h_small[5];
    {
        const int64_t nt = g->n_tasks, ns = g->n_split > 0 ? g->n_split : 1;
        PMA_TRY(hipMalloc(&t_target, nt * i4));
        PMA_TRY(hipMalloc(&t_begin, nt * i4));
        PMA_TRY(hipMalloc(&t_end, nt * i4));
        PMA_TRY(hipMalloc(&t_slot, nt * i4));
        PMA_TRY(hipMalloc(&t_split, nt * i4));
        PMA_TRY(hipMalloc(&t_key, nt * i4));
        PMA_TRY(hipMalloc(&tperm, nt * i4));
        PMA_TRY(hipMalloc(&tperm_tmp, nt * i4));
        PMA_TRY(hipMalloc(&g->task_target, nt * i4));
        PMA_TRY(hipMalloc(&g->task_begin, nt * i4));
        PMA_TRY(hipMalloc(&g->task_end, nt * i4));
        PMA_TRY(hipMalloc(&g->task_slot, nt * i4));
        PMA_TRY(hipMalloc(&g->task_split, nt * i4));
        PMA_TRY(hipMalloc(&g->split_target, ns * i4));
        PMA_TRY(hipMalloc(&g->split_slot0, ns * i4));
        PMA_TRY(hipMalloc(&g->split_count, ns * i4));
        int32_t *sc = nullptr;
        const int64_t ntt = (nt + kTile - 1) / kTile;
        PMA_TRY(hipMalloc(&sc, 256 * ntt * i4));
        split_fill_kernel<<<grid_for(L, 256), 256, 0, stream>>>(
            g->row_ptr, L, chunk, piece_base, slot_base, split_base, t_target, t_begin, t_end,
            t_slot, t_split, t_key, g->split_target, g->split_slot0, g->split_count);
        iota_kernel<<<grid_for(nt, 256), 256, 0, stream>>>(tperm, nt);
        hipError_t e = radix_sort_perm(t_key, bits_for(chunk >> kLenBucketShift), tperm, tperm_tmp, nt, sc, scan_tmp,
                                       stream);
        if (e == hipSuccess) {
            gather5_kernel<<<grid_for(nt, 256), 256, 0, stream>>>(
                tperm, nt, t_target, t_begin, t_end, t_slot, t_split, g->task_target,
                g->task_begin, g->task_end, g->task_slot, g->task_split);
            e = hipGetLastError();
        }
        if (e == hipSuccess)
            e = hipStreamSynchronize(stream);
        (void)hipFree(sc);
        if (e != hipSuccess) {
            snprintf(err, errlen, "work split: %s", hipGetErrorString(e));
            st = PMA_E_DEVICE;
            goto fail;
        }
    }
    goto done;

fail:
    (void)hipStreamSynchronize(stream);
    free_graph(g);
done:
    {
        int32_t *tmps[] = {d_src,     d_tgt,     perm,       perm_tmp,   counts,   scan_tmp,
                           small,     n_piece,    n_slot,     is_split, piece_base,
                           slot_base, split_base, t_target,  t_begin,    t_end,    t_slot,
                           t_split,   t_key,     tperm,      tperm_tmp, used,     kv_map};
        for (int32_t *p : tmps)
            if (p)
                (void)hipFree(p);
    }
    return st;
}

// Source-major view of the same edges, for the backward pass: positions of
// the target-grouped entries sorted stably by source (so by (source,
// target)), each entry's target, and per-source offsets.
__global__ void csc_fill(const int32_t *perm, const int32_t *csr_tgt, const int32_t *csr_eid,
                         int64_t nnz, int32_t *csc_tgt, int32_t *csc_eid)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < nnz) {
        csc_tgt[j] = csr_tgt[perm[j]];
        csc_eid[j] = csr_eid[perm[j]];
    }
}

// ---- banded source pieces --------------------------------------------------
// Sources with at least kBandMinDeg edges are cut at band boundaries, so that
// each of their pieces gathers target rows of one band only.
constexpr int kBandMinDeg = 64;

// band_start[k]: the first target whose CSR offset reaches ceil(k nnz / nb).
__global__ void band_bounds_kernel(const int32_t *row_ptr, int64_t L, int64_t nnz, int nb,
                                   int32_t *band_start)
{
    const int k = threadIdx.x;
    if (k > nb)
        return;
    if (k == 0 || k == nb) {
        band_start[k] = k == 0 ? 0 : (int32_t)L;
        return;
    }
    const int64_t goal = (nnz * k + nb - 1) / nb;
    int64_t lo = 0, hi = L;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (row_ptr[mid] >= goal)
            hi = mid;
        else
            lo = mid + 1;
    }
    band_start[k] = (int32_t)lo;
}

// first j in [b, e) with tgt[j] >= t (tgt ascending there)
__device__ inline int64_t lower_bound_t(const int32_t *tgt, int64_t b, int64_t e, int32_t t)
{
    while (b < e) {
        const int64_t mid = (b + e) >> 1;
        if (tgt[mid] >= t)
            e = mid;
        else
            b = mid + 1;
    }
    return b;
}

__device__ inline int64_t pieces_of(int64_t len, int chunk)
{
    return len > chunk ? (len + chunk - 1) / chunk : 1;
}

__global__ void src_piece_count(const int32_t *csc_ptr, const int32_t *csc_tgt,
                                const int32_t *band_start, int nb, int64_t S, int chunk, int32_t *n_piece,
                                int32_t *n_slot, int32_t *is_split, int32_t *n_long)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= S)
        return;
    const int64_t b = csc_ptr[s], e = csc_ptr[s + 1], g = e - b;
    if (g >= kBandMinDeg)
        atomicAdd(n_long, 1);
    int64_t n = 0;
    if (g < kBandMinDeg) {
        n = pieces_of(g, chunk);
    } else {
        for (int k = 0; k < nb; ++k) {
            const int64_t lo = lower_bound_t(csc_tgt, b, e, band_start[k]);
            const int64_t hi = lower_bound_t(csc_tgt, lo, e, band_start[k + 1]);
            if (hi > lo)
                n += pieces_of(hi - lo, chunk);
        }
    }
    n_piece[s] = (int32_t)n;
    n_slot[s] = n > 1 ? (int32_t)n : 0;
    is_split[s] = n > 1 ? 1 : 0;
}

// Pieces of source s at piece_base[s]: per band segment, ceil(len / chunk)
// even parts in target order. Sort key: band (L + 1), plus first target + 1
// for the pieces of long sources (short sources keep source order, first).
__global__ void src_piece_fill(const int32_t *csc_ptr, const int32_t *csc_tgt,
                               const int32_t *band_start, int sub, int64_t S, int64_t L,
                               int chunk, int banded,
                               const int32_t *piece_base, const int32_t *slot_base,
                               const int32_t *split_base, int32_t *u_source, int32_t *u_begin,
                               int32_t *u_end, int32_t *u_slot, int32_t *u_key,
                               int32_t *ss_source, int32_t *ss_slot0, int32_t *ss_count)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= S)
        return;
    const int64_t b = csc_ptr[s], e = csc_ptr[s + 1], g = e - b;
    const int64_t pb = piece_base[s];
    int64_t j = 0;
    // band k runs on XCD k mod kBands as its (k / kBands)-th sub-band
    auto emit = [&](int64_t sb, int64_t se, int band, bool by_target) {
        const int64_t xkey = (int64_t)(band % kBands) * sub + band / kBands;
        const int64_t len = se - sb, n = pieces_of(len, chunk);
        for (int64_t i = 0; i < n; ++i) {
            const int64_t pbeg = sb + (i * len) / n, pend = sb + ((i + 1) * len) / n;
            u_source[pb + j] = (int32_t)s;
            u_begin[pb + j] = (int32_t)pbeg;
            u_end[pb + j] = (int32_t)pend;
            u_key[pb + j] = (int32_t)(xkey * (L + 1) + (by_target && pend > pbeg ? csc_tgt[pbeg] + 1 : 0));
            ++j;
        }
    };
    if (g < kBandMinDeg)   // short rows: spread over the bands, source order
        emit(b, e, banded ? (int)(s % kBands) : 0, false);
    else {
        for (int k = 0; k < kBands * sub; ++k) {
            const int64_t lo = lower_bound_t(csc_tgt, b, e, band_start[k]);
            const int64_t hi = lower_bound_t(csc_tgt, lo, e, band_start[k + 1]);
            if (hi > lo)
                emit(lo, hi, k, true);
        }
    }
    for (int64_t i = 0; i < j; ++i)
        u_slot[pb + i] = j > 1 ? (int32_t)(slot_base[s] + i) : -1;
    if (j > 1) {
        const int32_t k = split_base[s];
        ss_source[k] = (int32_t)s;
        ss_slot0[k] = slot_base[s];
        ss_count[k] = (int32_t)j;
    }
}

// band_off[x] = first sorted piece of XCD x (key at least x sub (L + 1))
__global__ void band_off_kernel(const int32_t *key, int64_t n, int64_t L, int sub,
                                int32_t *band_off)
{
    const int k = threadIdx.x;
    if (k > kBands)
        return;
    const int64_t goal = (int64_t)k * sub * (L + 1);
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (key[mid] >= goal)
            hi = mid;
        else
            lo = mid + 1;
    }
    band_off[k] = (int32_t)lo;
}

pma_status build_csc(GraphDev *g, int64_t nnz, int64_t L, int64_t S, int chunk, int sub,
                     hipStream_t stream, char *err, size_t errlen)
{
    // sort keys (sub-band, target) stay below 2^31
    while (sub > 1 && (int64_t)kBands * sub * (L + 1) >= ((int64_t)1 << 31))
        sub >>= 1;
    const int nb = kBands * sub;
    pma_status st = PMA_OK;
    const size_t i4 = sizeof(int32_t);
    const int64_t n_sort = std::max(nnz, S);
    const int64_t ntiles = (n_sort + kTile - 1) / kTile;
    const int64_t count_len = 256 * ntiles;
    const int64_t scan_len = (count_len > n_sort ? count_len : n_sort) / kTile + 2;
    int32_t *perm = nullptr, *perm_tmp = nullptr, *counts = nullptr, *scan_tmp = nullptr,
            *small = nullptr, *n_piece = nullptr, *n_slot = nullptr,
            *is_split = nullptr, *piece_base = nullptr, *slot_base = nullptr,
            *split_base = nullptr, *band_start = nullptr;
    int32_t *u_source = nullptr, *u_begin = nullptr, *u_end = nullptr, *u_slot = nullptr,
            *u_key = nullptr, *s_key = nullptr, *tperm = nullptr, *tperm_tmp = nullptr,
            *sc = nullptr;
    int32_t h_small[8 + kBands + 1] = {0};
    PMA_TRY(hipMalloc(&perm, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMalloc(&perm_tmp, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMalloc(&counts, count_len * i4));
    PMA_TRY(hipMalloc(&scan_tmp, scan_len * i4));
    PMA_TRY(hipMalloc(&small, (8 + kBands + 1) * i4));
    PMA_TRY(hipMalloc(&n_piece, S * i4));
    PMA_TRY(hipMalloc(&n_slot, S * i4));
    PMA_TRY(hipMalloc(&is_split, S * i4));
    PMA_TRY(hipMalloc(&piece_base, S * i4));
    PMA_TRY(hipMalloc(&slot_base, S * i4));
    PMA_TRY(hipMalloc(&split_base, S * i4));
    PMA_TRY(hipMalloc(&band_start, (nb + 1) * i4));
    PMA_TRY(hipMalloc(&g->csc_ptr, (S + 1) * i4));
    PMA_TRY(hipMalloc(&g->csc_tgt, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMemsetAsync(g->csc_tgt + nnz, 0, kSrcPad * i4, stream));
    PMA_TRY(hipMalloc(&g->csc_eid, (nnz + kSrcPad) * i4));
    PMA_TRY(hipMemsetAsync(g->csc_eid + nnz, 0, kSrcPad * i4, stream));
    PMA_TRY(hipMemsetAsync(small, 0, (8 + kBands + 1) * i4, stream));
    iota_kernel<<<grid_for(nnz, 256), 256, 0, stream>>>(perm, nnz);
    PMA_TRY(radix_sort_perm(g->csr_src, bits_for(S - 1), perm, perm_tmp, nnz, counts, scan_tmp,
                            stream));
    PMA_TRY(hipMemsetAsync(perm + nnz, 0, kSrcPad * i4, stream));
    csc_fill<<<grid_for(nnz, 256), 256, 0, stream>>>(perm, g->csr_tgt, g->csr_eid, nnz,
                                                     g->csc_tgt, g->csc_eid);
    bounds_kernel<<<grid_for(S + 1, 256), 256, 0, stream>>>(g->csr_src, perm, nnz, S, g->csc_ptr);
    g->csc_pos = perm;   // kept
    perm = nullptr;
    // pieces per source: band segments, each in pieces of at most chunk
    band_bounds_kernel<<<1, 1024, 0, stream>>>(g->row_ptr, L, nnz, nb, band_start);
    src_piece_count<<<grid_for(S, 256), 256, 0, stream>>>(g->csc_ptr, g->csc_tgt, band_start, nb, S,
                                                          chunk, n_piece, n_slot, is_split,
                                                          small + 4);
    PMA_TRY(scan_exclusive(n_piece, piece_base, S, small + 1, scan_tmp, stream));
    PMA_TRY(scan_exclusive(n_slot, slot_base, S, small + 2, scan_tmp, stream));
    PMA_TRY(scan_exclusive(is_split, split_base, S, small + 3, scan_tmp, stream));
    PMA_TRY(hipGetLastError());
    PMA_TRY(hipMemcpyAsync(h_small, small, 8 * i4, hipMemcpyDeviceToHost, stream));
    PMA_TRY(hipStreamSynchronize(stream));
    g->n_stasks = h_small[1];
    g->n_sslots = h_small[2];
    g->n_ssplit = h_small[3];
    // Bands only pay where some source has long rows (whose pieces share
    // target rows); otherwise one band in source order.
    g->s_banded = h_small[4] > 0;
    {
        const int64_t nt = g->n_stasks, ns = g->n_ssplit > 0 ? g->n_ssplit : 1;
        const int64_t ntt = (nt + kTile - 1) / kTile;
        PMA_TRY(hipMalloc(&g->s_source, nt * i4));
        PMA_TRY(hipMalloc(&g->s_begin, nt * i4));
        PMA_TRY(hipMalloc(&g->s_end, nt * i4));
        PMA_TRY(hipMalloc(&g->s_slot, nt * i4));
        PMA_TRY(hipMalloc(&g->ss_source, ns * i4));
        PMA_TRY(hipMalloc(&g->ss_slot0, ns * i4));
        PMA_TRY(hipMalloc(&g->ss_count, ns * i4));
        PMA_TRY(hipMalloc(&u_source, nt * i4));
        PMA_TRY(hipMalloc(&u_begin, nt * i4));
        PMA_TRY(hipMalloc(&u_end, nt * i4));
        PMA_TRY(hipMalloc(&u_slot, nt * i4));
        PMA_TRY(hipMalloc(&u_key, nt * i4));
        PMA_TRY(hipMalloc(&s_key, nt * i4));
        PMA_TRY(hipMalloc(&tperm, nt * i4));
        PMA_TRY(hipMalloc(&tperm_tmp, nt * i4));
        PMA_TRY(hipMalloc(&sc, 256 * ntt * i4));
        src_piece_fill<<<grid_for(S, 256), 256, 0, stream>>>(
            g->csc_ptr, g->csc_tgt, band_start, sub, S, L, chunk, g->s_banded ? 1 : 0, piece_base,
            slot_base, split_base, u_source, u_begin, u_end, u_slot, u_key, g->ss_source,
            g->ss_slot0, g->ss_count);
        // order: band, then first target (stable)
        iota_kernel<<<grid_for(nt, 256), 256, 0, stream>>>(tperm, nt);
        PMA_TRY(radix_sort_perm(u_key, bits_for((int64_t)nb * (L + 1)), tperm, tperm_tmp, nt,
                                sc, scan_tmp, stream));
        gather5_kernel<<<grid_for(nt, 256), 256, 0, stream>>>(
            tperm, nt, u_source, u_begin, u_end, u_slot, u_key, g->s_source, g->s_begin, g->s_end,
            g->s_slot, s_key);
        band_off_kernel<<<1, 64, 0, stream>>>(s_key, nt, L, sub, small + 8);
        PMA_TRY(hipGetLastError());
        PMA_TRY(hipMemcpyAsync(h_small + 8, small + 8, (kBands + 1) * i4, hipMemcpyDeviceToHost,
                               stream));
        PMA_TRY(hipStreamSynchronize(stream));
        for (int k = 0; k <= kBands; ++k)
            g->s_band_off[k] = h_small[8 + k];
    }
    goto done;
fail:
    (void)hipStreamSynchronize(stream);
    {
        int32_t **own[] = {&g->csc_ptr,  &g->csc_tgt, &g->csc_pos,  &g->csc_eid,  &g->s_source, &g->s_begin,
                           &g->s_end,    &g->s_slot,  &g->ss_source, &g->ss_slot0, &g->ss_count};
        for (int32_t **q : own) {
            if (*q)
                (void)hipFree(*q);
            *q = nullptr;
        }
        g->n_stasks = g->n_ssplit = g->n_sslots = 0;
    }
done:
    for (int32_t *q : {perm, perm_tmp, counts, scan_tmp, small, n_piece, n_slot, is_split,
                       piece_base, slot_base, split_base, band_start, u_source, u_begin, u_end,
                       u_slot, u_key, s_key, tperm, tperm_tmp, sc})
        if (q)
            (void)hipFree(q);
    return st;
}

}  // namespace pma
