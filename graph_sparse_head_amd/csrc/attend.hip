// The whole per-target forward in one kernel: q projection, scores, online
// softmax and mix over the live edges, and out_proj (kpnn2
// PackedMultiheadAttention page, "Notes" steps 1-5, and the paragraph on
// queries with no live keys). Keys and values come from a separate projection
// launch (one source row serves many targets, so projecting it once is
// cheaper than once per edge).
//
// Lane layout. One wavefront handles one piece of a target's edge list for 16
// samples: lane l owns sample n = l % 16 and the channel slice
// [g * E/4, (g + 1) * E/4) with g = l / 16. With the weight tile as the MFMA
// "A" operand and the tokens as "B", a 16x16 MFMA output holds, in lane l,
// four rows of column l % 16. Two permutations make that column the lane's
// own sample and those rows the lane's own channels:
//   * the contraction index: at k-step ks, lane group g feeds physical
//     channels g * E/4 + (ks-th slice), i.e. exactly the slice it owns, and
//     the weight operand is read with the same permutation (any permutation
//     of k shared by A and B leaves the sum unchanged);
//   * the output rows: MFMA row r of n-tile nt is output channel
//     (E/4) * (r / 4) + 4 * nt + r % 4, so rows 4g .. 4g+3, which land in lane
//     group g, are channels of g's own slice.
// So q = x Wq^T + bq arrives in the lanes that score with it, and
// out = mixed Wo^T + bo is computed from the lanes that hold mixed, with no
// data exchanged between lanes. A head of d <= E/4 channels lies inside one
// lane, so its dot product needs no cross-lane reduction.
//
// A target longer than the plan's chunk is split into pieces; each piece
// stores its running (max, sum, partial mix), and merge_out, launched next,
// combines them in piece order and runs out_proj. (A last-piece-merges
// scheme needs agent-scope release/acquire fences, which write back and
// invalidate the L2 of an XCD each time; measured, it was slower.)
#include <math.h>

#include "pma_internal.h"

namespace pma {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

struct FusedK {
    const int32_t *csr_src;
    const int32_t *task_target, *task_begin, *task_end, *task_slot, *task_split;
    const int32_t *split_target, *split_slot0, *split_count;
    int64_t n_tasks, n_split;
    int B, L, H, passes;
    int64_t nnz;
    float scale;         // log2(e) / sqrt(d)
    const void *xq;      // (B, L, E) query tokens
    const void *wq, *bq, *wo, *bo;
    const void *kv;      // [S][2][B][E]
    void *out;           // (B, L, E)
    float *part_acc;     // [slot][B][E]
    float *part_ml;      // [slot][B][H][2]
    float *stat_ml;      // [L][B][H][2] or nullptr
    float *scores;       // [nnz][B][H] or nullptr
};

typedef __attribute__((ext_vector_type(2))) float f32x2;

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t word(const uint4 &u, int k)
{
    return k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
}
// element i of a run of 16-byte words holding T values, as fp32
template <typename T> __device__ inline float elem(const uint4 *w, int i)
{
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(word(w[i >> 2], i & 3));
    } else {
        const uint32_t x = word(w[i >> 3], (i >> 1) & 3);
        return (i & 1) ? bf_hi(x) : bf_lo(x);
    }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// y[c] for the lane's E/4 channels of its sample = x W^T + b, with the lane's
// own slice of x in xs (E/4 values of T as 16-byte words).
template <typename T, int E>
__device__ inline void project(const uint4 *xs, const T *W, const T *bias, int lane, float *y)
{
    constexpr int CPL = E / 4;
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int nt = 0; nt < E / 16; ++nt) {
        const int orow = CPL * (r >> 2) + 4 * nt + (r & 3);
        const T *wr = W + orow * E + g * CPL;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < CPL / 8; ++ks) {
                const uint4 wa = *reinterpret_cast<const uint4 *>(wr + 8 * ks);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa),
                                                              __builtin_bit_cast(bf16x8, xs[ks]),
                                                              acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int w = 0; w < CPL / 4; ++w) {
                const float4 wa = *reinterpret_cast<const float4 *>(wr + 4 * w);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa.x, __uint_as_float(xs[w].x), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa.y, __uint_as_float(xs[w].y), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa.z, __uint_as_float(xs[w].z), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa.w, __uint_as_float(xs[w].w), acc, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float bv = 0.f;
            if (bias) {
                if constexpr (sizeof(T) == 2)
                    bv = __uint_as_float((uint32_t)bias[g * CPL + 4 * nt + i] << 16);
                else
                    bv = bias[g * CPL + 4 * nt + i];
            }
            y[4 * nt + i] = acc[i] + bv;
        }
    }
}

// Pack n fp32 values into 16-byte words of T (bf16: round to nearest even).
template <typename T, int N> __device__ inline void pack(const float *v, uint4 *w)
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
            w[k] = make_uint4(__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                              __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3]));
    } else {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            uint32_t x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = pack_bf16(v[8 * k + 2 * j], v[8 * k + 2 * j + 1]);
            w[k] = make_uint4(x[0], x[1], x[2], x[3]);
        }
    }
}

// Steps 4 (end) and 5 for one (target, sample) row slice: mixed = acc / sum
// (zeros without edges), optional final (max, sum), out = mixed Wo^T + bo.
template <typename T, int E, int D>
__device__ inline void finish(const FusedK &a, int t, int b, bool valid, int lane,
                              const float *m, const float *l, const float *acc)
{
    constexpr int CPL = E / 4;
    constexpr int HL = D <= CPL ? CPL / D : 1;
    constexpr int GH = D <= CPL ? 1 : D / CPL;
    constexpr int HC = D <= CPL ? D : CPL;
    constexpr int VPL = CPL * (int)sizeof(T) / 16;
    constexpr int EPW = 16 / (int)sizeof(T);
    const int g = lane >> 4;
    const int B = a.B;
    const int c0 = g * CPL;
    const int h0 = GH == 1 ? g * HL : g / GH;
    const bool head_lead = GH == 1 || (g % GH) == 0;
    // ---- step 4 end: mixed = acc / sum (zeros without edges)
    float mix[CPL];
#pragma unroll
    for (int j = 0; j < HL; ++j)
#pragma unroll
        for (int i = 0; i < HC; ++i)
            mix[j * HC + i] = l[j] > 0.f ? acc[j * HC + i] / l[j] : 0.f;
    if (a.stat_ml && valid && head_lead) {
#pragma unroll
        for (int j = 0; j < HL; ++j) {
            float *st = a.stat_ml + (((int64_t)t * B + b) * a.H + h0 + j) * 2;
            st[0] = m[j];
            st[1] = l[j];
        }
    }

    // ---- step 5: out = mixed Wo^T + bo
    uint4 ms[VPL];
    pack<T, CPL>(mix, ms);
    float o[CPL];
    project<T, E>(ms, reinterpret_cast<const T *>(a.wo), reinterpret_cast<const T *>(a.bo), lane, o);
    if (valid) {
        uint4 ow[VPL];
        pack<T, CPL>(o, ow);
        T *dst = reinterpret_cast<T *>(a.out) + ((int64_t)b * a.L + t) * E + c0;
#pragma unroll
        for (int w = 0; w < VPL; ++w)
            *reinterpret_cast<uint4 *>(dst + w * EPW) = ow[w];
    }
}

template <typename T, int E, int D, int U>
__global__ void __launch_bounds__(256) attend_fused(FusedK a)
{
    constexpr int CPL = E / 4;                   // channels per lane
    constexpr int HL = D <= CPL ? CPL / D : 1;   // heads inside one lane
    constexpr int GH = D <= CPL ? 1 : D / CPL;   // lane groups per head
    constexpr int HC = D <= CPL ? D : CPL;       // channels of one head inside the lane
    constexpr int VPL = CPL * (int)sizeof(T) / 16;
    constexpr int EPW = 16 / (int)sizeof(T);     // elements per 16-byte word
    constexpr bool BF = sizeof(T) == 2;

    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= a.n_tasks * a.passes)
        return;
    const int64_t task = unit / a.passes;
    const int pass = (int)(unit - task * a.passes);
    const int t = a.task_target[task];
    const int beg = a.task_begin[task], end = a.task_end[task];
    const int slot = a.task_slot[task];
    const int g = lane >> 4, n = lane & 15;
    const int B = a.B;
    const int b = pass * 16 + n;
    const bool valid = b < B;
    const int c0 = g * CPL;
    const int h0 = GH == 1 ? g * HL : g / GH;    // first head of the lane
    const bool head_lead = GH == 1 || (g % GH) == 0;

    // ---- step 1: q for (b, t), this lane's channels
    float qf[CPL];
    {
        uint4 xs[VPL];
        const T *xr = reinterpret_cast<const T *>(a.xq) + ((int64_t)b * a.L + t) * E + c0;
#pragma unroll
        for (int w = 0; w < VPL; ++w)
            xs[w] = valid ? *reinterpret_cast<const uint4 *>(xr + w * EPW) : make_uint4(0, 0, 0, 0);
        project<T, E>(xs, reinterpret_cast<const T *>(a.wq), reinterpret_cast<const T *>(a.bq),
                      lane, qf);
    }
    // bf16: q rounded to bf16 and dotted with bf16 keys (v_dot2); fp32: q pre-scaled
    uint32_t qb[BF ? CPL / 2 : 1];
    if constexpr (BF) {
#pragma unroll
        for (int i = 0; i < CPL / 2; ++i)
            qb[i] = pack_bf16(qf[2 * i], qf[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) qf[i] *= a.scale;
    }

    // ---- steps 2-4: scores, online softmax, mix
    float m[HL], l[HL], acc[CPL];
#pragma unroll
    for (int j = 0; j < HL; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    const int64_t row2 = (int64_t)2 * B * E, voff = (int64_t)B * E;
    const T *kvl = reinterpret_cast<const T *>(a.kv) + (int64_t)b * E + c0;

    for (int p = beg; p < end; p += U) {
        const int nu = end - p < U ? end - p : U;
        uint4 kk[U][VPL], vv[U][VPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = a.csr_src[u < nu ? p + u : p];
            const T *kr = kvl + (int64_t)s * row2;
#pragma unroll
            for (int w = 0; w < VPL; ++w) {
                kk[u][w] = valid ? *reinterpret_cast<const uint4 *>(kr + w * EPW) : make_uint4(0, 0, 0, 0);
                vv[u][w] = valid ? *reinterpret_cast<const uint4 *>(kr + voff + w * EPW) : make_uint4(0, 0, 0, 0);
            }
        }
        float sc[U][HL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < HL; ++j) {
                float dot = 0.f;
                if constexpr (BF) {
#pragma unroll
                    for (int i = 0; i < HC / 2; ++i) {
                        const int e = j * HC + 2 * i;          // even element index
                        dot = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2, qb[e / 2]),
                            __builtin_bit_cast(bf16x2, word(kk[u][e / 8], (e / 2) & 3)), dot, false);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < HC; ++i)
                        dot = fmaf(qf[j * HC + i], elem<T>(kk[u], j * HC + i), dot);
                }
                if constexpr (GH >= 2) dot += __shfl_xor(dot, 16, 64);
                if constexpr (GH >= 4) dot += __shfl_xor(dot, 32, 64);
                if constexpr (BF) dot *= a.scale;
                sc[u][j] = u < nu ? dot : -INFINITY;
            }
        }
        if (a.scores && valid && head_lead) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nu) {
#pragma unroll
                    for (int j = 0; j < HL; ++j)
                        a.scores[((int64_t)(p + u) * B + b) * a.H + h0 + j] = sc[u][j];
                }
        }
#pragma unroll
        for (int j = 0; j < HL; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
            const float alpha = fast_exp2(m[j] - mx);
            l[j] *= alpha;
#pragma unroll
            for (int i = 0; i < HC; ++i) acc[j * HC + i] *= alpha;
            m[j] = mx;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < HL; ++j) {
                const float pe = fast_exp2(sc[u][j] - m[j]);
                l[j] += pe;
#pragma unroll
                for (int i = 0; i < HC; ++i)
                    acc[j * HC + i] = fmaf(pe, elem<T>(vv[u], j * HC + i), acc[j * HC + i]);
            }
        }
    }

    // ---- a piece of a split target leaves (max, sum, partial mix) for merge_out
    if (slot >= 0) {
        if (valid) {
            float *pa = a.part_acc + ((int64_t)slot * B + b) * E + c0;
#pragma unroll
            for (int k = 0; k < CPL / 4; ++k)
                reinterpret_cast<float4 *>(pa)[k] =
                    make_float4(acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
            if (head_lead) {
#pragma unroll
                for (int j = 0; j < HL; ++j) {
                    float *pm = a.part_ml + (((int64_t)slot * B + b) * a.H + h0 + j) * 2;
                    pm[0] = m[j];
                    pm[1] = l[j];
                }
            }
        }
        return;
    }

    finish<T, E, D>(a, t, b, valid, lane, m, l, acc);
}

// Merge the pieces of each split target in piece order, then out_proj.
// One wavefront per (split target, 16 samples), lanes as in attend_fused.
template <typename T, int E, int D>
__global__ void __launch_bounds__(256) merge_out(FusedK a)
{
    constexpr int CPL = E / 4;
    constexpr int HL = D <= CPL ? CPL / D : 1;
    constexpr int GH = D <= CPL ? 1 : D / CPL;
    constexpr int HC = D <= CPL ? D : CPL;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= a.n_split * a.passes)
        return;
    const int k = (int)(unit / a.passes);
    const int pass = (int)(unit - (int64_t)k * a.passes);
    const int g = lane >> 4, n = lane & 15;
    const int B = a.B;
    const int b = pass * 16 + n;
    const bool valid = b < B;
    const int c0 = g * CPL;
    const int h0 = GH == 1 ? g * HL : g / GH;
    const int t = a.split_target[k], s0 = a.split_slot0[k], np = a.split_count[k];
    float m[HL], l[HL], acc[CPL];
#pragma unroll
    for (int j = 0; j < HL; ++j) {
        float M = -INFINITY;
        for (int q = 0; q < np && valid; ++q)
            M = fmaxf(M, a.part_ml[(((int64_t)(s0 + q) * B + b) * a.H + h0 + j) * 2]);
        m[j] = M;
        l[j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    for (int q = 0; q < np && valid; ++q) {
        const float4 *pq = reinterpret_cast<const float4 *>(
            a.part_acc + ((int64_t)(s0 + q) * B + b) * E + c0);
#pragma unroll
        for (int j = 0; j < HL; ++j) {
            const float2 ml = *reinterpret_cast<const float2 *>(
                a.part_ml + (((int64_t)(s0 + q) * B + b) * a.H + h0 + j) * 2);
            const float w = fast_exp2(ml.x - m[j]);
            l[j] = fmaf(ml.y, w, l[j]);
#pragma unroll
            for (int i4 = 0; i4 < HC / 4; ++i4) {
                const float4 v = pq[(j * HC) / 4 + i4];
                const int i = j * HC + 4 * i4;
                acc[i] = fmaf(v.x, w, acc[i]);
                acc[i + 1] = fmaf(v.y, w, acc[i + 1]);
                acc[i + 2] = fmaf(v.z, w, acc[i + 2]);
                acc[i + 3] = fmaf(v.w, w, acc[i + 3]);
            }
        }
    }
    finish<T, E, D>(a, t, b, valid, lane, m, l, acc);
}

template <typename T, int E, int D, int U>
hipError_t run(const FusedK &k, hipStream_t s)
{
    const int64_t units = k.n_tasks * k.passes;
    attend_fused<T, E, D, U><<<(unsigned)((units + 3) / 4), 256, 0, s>>>(k);
    return hipGetLastError();
}

template <typename T, int E, int D>
hipError_t run_merge(const FusedK &k, hipStream_t s)
{
    const int64_t units = k.n_split * k.passes;
    merge_out<T, E, D><<<(unsigned)((units + 3) / 4), 256, 0, s>>>(k);
    return hipGetLastError();
}

template <typename T, int E>
hipError_t dispatch_d(const FusedK &k, int d, bool merge, hipStream_t s)
{
    constexpr int U = (E * (int)sizeof(T) <= 128) ? 4 : (E * (int)sizeof(T) <= 256 ? 2 : 1);
    switch (d) {
    case 8: return merge ? run_merge<T, E, 8>(k, s) : run<T, E, 8, U>(k, s);
    case 16: return merge ? run_merge<T, E, 16>(k, s) : run<T, E, 16, U>(k, s);
    case 32: return merge ? run_merge<T, E, 32>(k, s) : run<T, E, 32, U>(k, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fused_supported(int64_t E, int64_t H, pma_dtype dt)
{
    if (E != 64 && E != 128)
        return false;
    const int64_t d = E / H;
    if (d != 8 && d != 16 && d != 32)
        return false;
    // a head spans at most 4 lane groups; d >= 8 keeps bf16 words whole
    return dt == PMA_BF16 || dt == PMA_F32;
}

pma_status launch_fused(const FusedArgs &x, bool merge, hipStream_t s)
{
    FusedK k;
    const GraphDev *g = x.g;
    k.csr_src = g->csr_src;
    k.task_target = g->task_target;
    k.task_begin = g->task_begin;
    k.task_end = g->task_end;
    k.task_slot = g->task_slot;
    k.task_split = g->task_split;
    k.split_slot0 = g->split_slot0;
    k.split_count = g->split_count;
    k.n_tasks = g->n_tasks;
    k.B = (int)x.B;
    k.L = (int)x.L;
    k.H = (int)x.H;
    k.passes = (int)((x.B + 15) / 16);
    k.nnz = x.nnz;
    const int d = (int)(x.E / x.H);
    k.scale = (float)(1.4426950408889634 / sqrt((double)d));
    k.xq = x.xq;
    k.wq = x.wq;
    k.bq = x.bq;
    k.wo = x.wo;
    k.bo = x.bo;
    k.kv = x.kv;
    k.out = x.out;
    k.part_acc = x.part_acc;
    k.part_ml = x.part_ml;
    k.stat_ml = x.stat_ml;
    k.scores = x.scores;
    hipError_t e;
    k.n_split = g->n_split;
    k.split_target = g->split_target;
    if (merge && k.n_split == 0)
        return PMA_OK;
    if (x.dt == PMA_BF16)
        e = x.E == 64 ? dispatch_d<uint16_t, 64>(k, d, merge, s)
                      : dispatch_d<uint16_t, 128>(k, d, merge, s);
    else
        e = x.E == 64 ? dispatch_d<float, 64>(k, d, merge, s) : dispatch_d<float, 128>(k, d, merge, s);
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
