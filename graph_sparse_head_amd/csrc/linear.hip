// PackedLinear on the same packed pairs (kpnn2 PackedMultiheadAttention page,
// "See also": one trained scalar per edge, the same for every sample,
// information flowing from source to target): a linear map whose weight
// matrix (L targets x S sources) holds a learned scalar w_e at each live
// pair and zero elsewhere,
//   y[b, t, c] = bias[t] + sum over edges e into t of w_e x[b, s_e, c],
// for every sample b and channel c (one channel for a plain nn.Linear-shaped
// layer). Its gradients:
//   dx[b, s, c] = sum over edges e out of s of w_e dy[b, t_e, c],
//   dw_e = sum over b, c of dy[b, t_e, c] x[b, s_e, c],  dbias[t] = sum over b, c of dy[b, t, c].
//
// A node's "row" is all its samples' channels, R = B C values, each a
// segment of C at stride sb (batch-first tensors: sb = nodes x C). When C
// fills whole 16-byte chunks the kernels read the caller's batch-first
// tensors directly; otherwise the batch goes node-major first (one
// contiguous row per node, transposed to and from through LDS tiles;
// nothing to do for B = 1), so that an edge reads one contiguous row for
// the whole batch instead of B scattered values. The product walks the target
// pieces of the attention's index (edges by target); the input gradient the
// source pieces of its source-major view: one kernel, rows swapped. One
// wavefront takes a piece (or a 64-chunk segment of a long row): each lane
// owns one chunk of the row (16 bytes when R allows, else one value) for
// every G-th edge of the piece, G = 64 / lanes per row, and the G partial
// sums meet through lane shuffles. Split pieces write fp32 partials that a
// merge adds in slot order. Sums are fp32; outputs round to the plan dtype.
#include "pma_internal.h"

namespace pma {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
template <typename T> __device__ inline float ld(const T *p);
template <> __device__ inline float ld<float>(const float *p) { return *p; }
template <> __device__ inline float ld<uint16_t>(const uint16_t *p)
{
    return __uint_as_float((uint32_t)*p << 16);
}
template <typename T> __device__ inline void st(T *p, float x);
template <> __device__ inline void st<float>(float *p, float x) { *p = x; }
template <> __device__ inline void st<uint16_t>(uint16_t *p, float x)
{
    *p = (uint16_t)(pack_bf16(x, 0.f) & 0xffffu);
}

// VEC consecutive elements widened to fp32 (one 16-byte load when VEC > 1)
template <typename T, int VEC> __device__ inline void load_n(const T *p, float (&f)[VEC])
{
    if constexpr (VEC == 1) {
        f[0] = ld(p);
    } else {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = __uint_as_float(w[i] << 16);
                f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
}
template <typename T, int VEC> __device__ inline void store_n(T *p, const float (&f)[VEC])
{
    if constexpr (VEC == 1) {
        st(p, f[0]);
    } else if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                                                   __float_as_uint(f[2]), __float_as_uint(f[3]));
    } else {
        *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                                                   pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
    }
}

constexpr int kU = 4;   // edges per lane group loaded together

// Sum over the lanes that share lane % CGP (all 64 lanes active).
template <int VEC> __device__ inline void lane_sum(float (&a)[VEC], int cgp)
{
    for (int m = cgp; m < 64; m <<= 1)
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            a[i] += __shfl_xor(a[i], m, 64);
}

// Wavefront = (piece, segment of 64 chunks of the row). a.cgp = lanes per
// row segment (power of two), G = 64 / cgp edge groups.
template <typename T, int VEC, int U>
__global__ void __launch_bounds__(256) lin_wave(const LinArgs a)
{
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t task = wave / a.nseg;
    const int seg = (int)(wave - task * a.nseg);
    if (task >= a.n_tasks)
        return;   // whole wavefront
    const int nc = a.R / VEC;
    const int cg = seg * 64 + (lane & (a.cgp - 1));
    const int j = lane / a.cgp, G = 64 / a.cgp;
    const bool on = cg < nc;
    const int row = a.t_row[task], beg = a.t_begin[task], end = a.t_end[task];
    const int slot = a.t_slot[task];
    // chunk cg = (segment b, chunk within the segment)
    const int cpv = a.Cs / VEC;
    const int sb = (on ? cg : 0) / cpv, sc = (on ? cg : 0) - sb * cpv;
    const T *X = reinterpret_cast<const T *>(a.x) + (int64_t)sb * a.sb_in + sc * VEC;
    const T *W = reinterpret_cast<const T *>(a.w);
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        acc[i] = 0.f;
    // U edges of this lane's group per step (p0 + j + u G), the next U in
    // flight; entries past the piece's end read entry 0 of the piece and
    // count with weight 0
    float wv[U], wn[U], xv[U][VEC], xn[U][VEC];
    auto fetch = [&](int p0, float (&ww)[U], float (&xx)[U][VEC]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = p0 + u * G;
            const int qq = q < end ? q : beg;   // a valid entry; its weight is dropped
            const float wq = ld(W + a.eid[qq]);
            ww[u] = q < end ? wq : 0.f;
            load_n<T, VEC>(X + (int64_t)a.idx[qq] * a.sn_in, xx[u]);
        }
    };
    const int step = U * G;
    int p = beg + j;
    if (p < end)
        fetch(p, wv, xv);
    for (; p < end; p += step) {
        const bool more = p + step < end;
        if (more)
            fetch(p + step, wn, xn);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                acc[i] = fmaf(wv[u], xv[u][i], acc[i]);
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                wv[u] = wn[u];
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    xv[u][i] = xn[u][i];
            }
        }
    }
    lane_sum<VEC>(acc, a.cgp);
    if (j != 0 || !on)
        return;
    if (slot >= 0) {
        float *d = a.part + (int64_t)slot * a.R + cg * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            d[i] = acc[i];
        return;
    }
    if (a.bias) {
        const float bv = ld(reinterpret_cast<const T *>(a.bias) + row);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            acc[i] += bv;
    }
    store_n<T, VEC>(reinterpret_cast<T *>(a.y) + (int64_t)row * a.sn_out + (int64_t)sb * a.sb_out +
                        sc * VEC, acc);
}

// Batch-first rows whose segments (one sample's C channels) fill 16-byte
// chunks: thread = (piece, sample, chunk), chunks fastest, each walking the
// whole piece with kU edges loaded together and the next kU in flight. UNI:
// a piece's threads fill whole wavefronts (scalar index loads).
template <typename T, int VEC, bool UNI>
__global__ void __launch_bounds__(256) lin_thread(const LinArgs a)
{
    const int cpv = a.Cs / VEC;
    const int nb = a.R / a.Cs;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gb = idx / cpv;
    const int sc = (int)(idx - gb * cpv);
    int64_t task = gb / nb;
    const int sb = (int)(gb - task * nb);
    if (UNI)
        task = __builtin_amdgcn_readfirstlane((int)task);
    if (task >= a.n_tasks)
        return;
    const int row = a.t_row[task], beg = a.t_begin[task], end = a.t_end[task];
    const int slot = a.t_slot[task];
    const T *X = reinterpret_cast<const T *>(a.x) + (int64_t)sb * a.sb_in + sc * VEC;
    const T *W = reinterpret_cast<const T *>(a.w);
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        acc[i] = 0.f;
    float wv[kU], wn[kU], xv[kU][VEC], xn[kU][VEC];
    // entries past the piece's end (at most kU - 1, inside the index
    // arrays' zero padding) are loaded and not used
    auto fetch = [&](int p0, float (&ww)[kU], float (&xx)[kU][VEC]) {
        int src[kU], eid[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            src[u] = a.idx[p0 + u];
            eid[u] = a.eid[p0 + u];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            ww[u] = ld(W + eid[u]);
            load_n<T, VEC>(X + (int64_t)src[u] * a.sn_in, xx[u]);
        }
    };
    if (beg < end)
        fetch(beg, wv, xv);
    for (int p0 = beg; p0 < end; p0 += kU) {
        const bool more = p0 + kU < end;
        if (more)
            fetch(p0 + kU, wn, xn);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (p0 + u < end) {
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    acc[i] = fmaf(wv[u], xv[u][i], acc[i]);
            }
        if (more) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                wv[u] = wn[u];
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    xv[u][i] = xn[u][i];
            }
        }
    }
    const int r = sb * a.Cs + sc * VEC;
    if (slot >= 0) {
        float *d = a.part + (int64_t)slot * a.R + r;
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            d[i] = acc[i];
        return;
    }
    if (a.bias) {
        const float bv = ld(reinterpret_cast<const T *>(a.bias) + row);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            acc[i] += bv;
    }
    store_n<T, VEC>(reinterpret_cast<T *>(a.y) + (int64_t)row * a.sn_out + (int64_t)sb * a.sb_out +
                        sc * VEC, acc);
}

// Rows cut into pieces: the pieces' partials in slot order, plus the bias.
// Thread = (split row, element).
template <typename T>
__global__ void __launch_bounds__(256) lin_merge(const LinArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t i = idx / a.R;
    const int r = (int)(idx - i * a.R);
    if (i >= a.n_split)
        return;
    const int row = a.s_row[i], slot0 = a.s_slot0[i], count = a.s_count[i];
    float acc = 0.f;
    for (int k = 0; k < count; ++k)
        acc += a.part[(int64_t)(slot0 + k) * a.R + r];
    if (a.bias)
        acc += ld(reinterpret_cast<const T *>(a.bias) + row);
    const int sb = r / a.Cs;
    st(reinterpret_cast<T *>(a.y) + (int64_t)row * a.sn_out + (int64_t)sb * a.sb_out + (r - sb * a.Cs),
       acc);
}

// dw_e = dot(dy row of t_e, x row of s_e) over R; dbias[t] = sum of the dy
// row of t. A group of cgp lanes per edge (or target), chunks strided by
// cgp; rows laid out as in lin_wave (segments of Cs at strides sbx / sbg).
template <typename T, int VEC>
__global__ void __launch_bounds__(256) lin_rowdots(const RowDots a)
{
    const int64_t gid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / a.cgp;
    const int k = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) % a.cgp);
    const int nc = a.R / VEC, cpv = a.Cs / VEC;
    const bool is_edge = gid < a.nnz;
    const bool is_bias = !is_edge && a.db && gid - a.nnz < a.L;
    float acc = 0.f;
    if (is_edge || is_bias) {
        const int64_t t = is_edge ? a.csr_tgt[gid] : gid - a.nnz;
        const T *g = reinterpret_cast<const T *>(a.dy) + t * a.sng;
        const T *x = is_edge ? reinterpret_cast<const T *>(a.x) + (int64_t)a.csr_src[gid] * a.snx
                             : nullptr;
        for (int c = k; c < nc; c += a.cgp) {
            const int sb = c / cpv, sc = c - sb * cpv;
            float gv[VEC], xv[VEC];
            load_n<T, VEC>(g + (int64_t)sb * a.sbg + sc * VEC, gv);
            if (is_edge) {
                load_n<T, VEC>(x + (int64_t)sb * a.sbx + sc * VEC, xv);
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    acc = fmaf(gv[i], xv[i], acc);
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    acc += gv[i];
            }
        }
    }
    for (int m = 1; m < a.cgp; m <<= 1)
        acc += __shfl_xor(acc, m, 64);
    if (k != 0)
        return;
    if (is_edge)
        st(reinterpret_cast<T *>(a.dw) + a.csr_eid[gid], acc);
    else if (is_bias)
        st(reinterpret_cast<T *>(a.db) + (gid - a.nnz), acc);
}

// out[q][p][c] = in[p][q][c] for p < P, q < Q, c < C, through an LDS tile of
// TP x TQ items: reads are contiguous along q, writes along p.
template <typename T>
__global__ void __launch_bounds__(256) transpose_pqc(const T *in, T *out, int64_t P, int64_t Q,
                                                     int C, int TP, int TQ)
{
    extern __shared__ __attribute__((aligned(16))) char tl[];
    T *tile = reinterpret_cast<T *>(tl);
    const int64_t p0 = (int64_t)blockIdx.y * TP, q0 = (int64_t)blockIdx.x * TQ;
    const int rowlen = TQ * C;   // elements of one p row in the tile
    for (int i = threadIdx.x; i < TP * rowlen; i += blockDim.x) {
        const int pl = i / rowlen, off = i - pl * rowlen;
        const int64_t p = p0 + pl, q = q0 + off / C;
        if (p < P && q < Q)
            tile[i] = in[(p * Q + q0) * C + off];
    }
    __syncthreads();
    const int outlen = TP * C;   // elements of one q row of the output tile
    for (int i = threadIdx.x; i < TQ * outlen; i += blockDim.x) {
        const int ql = i / outlen, off = i - ql * outlen;
        const int pl = off / C, c = off - pl * C;
        const int64_t p = p0 + pl, q = q0 + ql;
        if (p < P && q < Q)
            out[(q * P + p0) * C + off] = tile[pl * rowlen + ql * C + c];
    }
}

inline unsigned grid(int64_t n) { return (unsigned)((n + 255) / 256); }

int pow2_at_least(int n)
{
    int p = 1;
    while (p < n)
        p <<= 1;
    return p;
}

template <typename T, int VEC>
void wave_launch(LinArgs a, hipStream_t s)
{
    const int nc = a.R / VEC;
    if (VEC > 1 && a.Cs < a.R) {
        // batch-first segments: a thread per chunk of each sample's segment
        const int64_t per = nc;   // threads per piece
        const int64_t n = a.n_tasks * per;
        if (per % 64 == 0)
            lin_thread<T, VEC, true><<<grid(n), 256, 0, s>>>(a);
        else
            lin_thread<T, VEC, false><<<grid(n), 256, 0, s>>>(a);
    } else {
        a.nseg = (nc + 63) / 64;
        a.cgp = nc >= 64 ? 64 : pow2_at_least(nc);
        // at most 64 edges of a piece per wavefront step: G x U <= 64
        if (a.cgp >= 4)
            lin_wave<T, VEC, 4><<<grid(a.n_tasks * a.nseg * 64), 256, 0, s>>>(a);
        else
            lin_wave<T, VEC, 1><<<grid(a.n_tasks * a.nseg * 64), 256, 0, s>>>(a);
    }
    if (a.n_split > 0)
        lin_merge<T><<<grid(a.n_split * a.R), 256, 0, s>>>(a);
}

template <typename T, int VEC>
void rowdots_launch(RowDots a, hipStream_t s)
{
    const int nc = a.R / VEC;
    a.cgp = nc >= 64 ? 64 : pow2_at_least(nc);
    const int64_t groups = a.nnz + (a.db ? a.L : 0);
    lin_rowdots<T, VEC><<<grid(groups * a.cgp), 256, 0, s>>>(a);
}

template <typename T>
hipError_t transpose_launch(const void *in, void *out, int64_t P, int64_t Q, int C, hipStream_t s)
{
    // TP x TQ items of C elements, at most 32 KB of LDS
    const int64_t items = (32 * 1024) / ((int64_t)C * sizeof(T));
    int T2 = 32;
    while (T2 > 1 && (int64_t)T2 * T2 > items)
        T2 >>= 1;
    if (items < 1)
        return hipErrorInvalidValue;
    const dim3 g((unsigned)((Q + T2 - 1) / T2), (unsigned)((P + T2 - 1) / T2));
    transpose_pqc<T><<<g, 256, (size_t)T2 * T2 * C * sizeof(T), s>>>(
        reinterpret_cast<const T *>(in), reinterpret_cast<T *>(out), P, Q, C, T2, T2);
    return hipGetLastError();
}

}  // namespace

int lin_vec(int64_t Cs, pma_dtype dt, const void *const *ptrs, int n)
{
    const int vec = dt == PMA_BF16 ? 8 : 4;
    uintptr_t bits = 0;
    for (int i = 0; i < n; ++i)
        bits |= (uintptr_t)ptrs[i];
    return Cs % vec == 0 && (bits & 15) == 0 ? vec : 1;
}

pma_status launch_spmm(const LinArgs &a, pma_dtype dt, int vec, hipStream_t s)
{
    if (dt == PMA_BF16) {
        if (vec > 1)
            wave_launch<uint16_t, 8>(a, s);
        else
            wave_launch<uint16_t, 1>(a, s);
    } else {
        if (vec > 1)
            wave_launch<float, 4>(a, s);
        else
            wave_launch<float, 1>(a, s);
    }
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status launch_lin_rowdots(const RowDots &a, pma_dtype dt, int vec, hipStream_t s)
{
    if (dt == PMA_BF16) {
        if (vec > 1)
            rowdots_launch<uint16_t, 8>(a, s);
        else
            rowdots_launch<uint16_t, 1>(a, s);
    } else {
        if (vec > 1)
            rowdots_launch<float, 4>(a, s);
        else
            rowdots_launch<float, 1>(a, s);
    }
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status launch_transpose(const void *in, void *out, int64_t P, int64_t Q, int64_t C,
                            pma_dtype dt, hipStream_t s)
{
    if (P <= 0 || Q <= 0 || C <= 0)
        return PMA_OK;
    const hipError_t e = dt == PMA_BF16 ? transpose_launch<uint16_t>(in, out, P, Q, (int)C, s)
                                        : transpose_launch<float>(in, out, P, Q, (int)C, s);
    return e == hipSuccess ? PMA_OK : (e == hipErrorInvalidValue ? PMA_E_UNSUPPORTED : PMA_E_DEVICE);
}

}  // namespace pma
