// The four nn.Linear projections of the layer (kpnn2 PackedMultiheadAttention
// page, "Notes" step 1 and step 5; the attribute table: four embed_dim ->
// embed_dim maps q_proj, k_proj, v_proj, out_proj): y = x W^T + b with W
// stored [out][in].
//
// One launch may apply up to three projections to the same input rows (the
// q, k and v maps when query, key and value are one tensor), each output
// block written to its own layout. The contraction runs on the matrix cores:
// with the weight tile as the MFMA "A" operand and the token rows as "B", each
// lane ends up holding four consecutive output channels of one token row,
// which it stores directly.
#include "pma_internal.h"

namespace pma {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ inline float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ inline uint16_t f2bf(float f) { return (uint16_t)(pack_bf16(f, 0.f) & 0xffffu); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kVec = 4;    // elements per 16-byte load
    static constexpr int kStep = 16;  // k covered by one 16-byte load per lane group
};
template <> struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    static constexpr int kStep = 32;
};

// Input row of iteration row r.
__device__ inline int64_t in_row(const ProjArgs &a, int64_t r)
{
    if (a.row_list) {   // batch-first input, iteration rows (sample, listed token)
        const int64_t b = r / a.n, i = r - b * a.n;
        return b * a.n_in + a.row_list[i];
    }
    if (a.x_token_major < 0 || a.x_token_major == a.token_major)
        return r;
    int64_t b, i;
    if (a.token_major) {
        i = r / a.B;
        b = r - i * a.B;
    } else {
        b = r / a.n;
        i = r - b * a.n;
    }
    return a.x_token_major ? i * a.B + b : b * a.n + i;
}

// (sample, token) of iteration row r
__device__ inline void decompose(const ProjArgs &a, int64_t r, int64_t &b, int64_t &i)
{
    if (a.token_major) {
        i = r / a.B;
        b = r - i * a.B;
    } else {
        b = r / a.n;
        i = r - b * a.n;
    }
}

// (b, i) of iteration row r + step, from (b, i) of row r
__device__ inline void advance(const ProjArgs &a, int64_t &b, int64_t &i, int step)
{
    if (a.token_major) {
        b += step;
        while (b >= a.B) {
            b -= a.B;
            ++i;
        }
    } else {
        i += step;
        while (i >= a.n) {
            i -= a.n;
            ++b;
        }
    }
}

__device__ inline int64_t out_offset(const ProjArgs &a, const ProjOut &o, uint32_t r)
{
    uint32_t b, i;
    if (a.token_major) {
        i = r / (uint32_t)a.B;
        b = r - i * (uint32_t)a.B;
    } else {
        b = r / (uint32_t)a.n;
        i = r - b * (uint32_t)a.n;
    }
    return (int64_t)b * o.sb + (int64_t)i * o.si;
}

// Persistent matrix-core projection. A workgroup of WAVES wavefronts first
// copies the weight tiles of all its output blocks into LDS, laid out in
// MFMA fragment order (one 1 KB fragment per (block, n-tile, k-step), lane l
// at byte 16 l), so every later fragment read is one conflict-free 16-byte
// LDS load, and the biases as fp32 after them. It then walks row tiles of
// WAVES x RG x 16 rows, stride gridDim. Each wavefront keeps its rows' x
// fragments in registers and loads the next tile's fragments before
// computing the current one. bf16 output blocks go through a per-wavefront
// LDS staging area so that stores are whole 16-byte chunks of whole rows;
// fp32 lanes already hold 16 contiguous bytes and store them directly.
template <typename T, int K, int RG, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) proj_mfma(ProjArgs a)
{
    constexpr int NKS = K / Elem<T>::kStep;
    constexpr int E = K;
    constexpr int NT = E / 16;
    constexpr int ROWS = RG * 16;
    constexpr int PITCH = E * (int)sizeof(T) + 16;       // bytes per staged row
    constexpr int CPR = E * (int)sizeof(T) / 16;         // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                        // rows stored per instruction
    // bf16 results go through a per-wavefront LDS staging area so that stores
    // are whole 16-byte chunks of whole rows; an fp32 lane already holds 16
    // contiguous bytes of its row and stores them directly.
    constexpr bool STAGE = sizeof(T) == 2;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int nblk = a.nblk;
    char *wl = lds;                                      // nblk * NT * NKS KB
    // the biases as fp32 (zeros without bias) after the fragments, so that
    // the compute loop reads no global memory besides the x prefetch
    float *bl = reinterpret_cast<float *>(lds + nblk * NT * NKS * 1024);
    char *stage = lds + nblk * NT * NKS * 1024 + nblk * E * 4 + (threadIdx.x >> 6) * (ROWS * PITCH);
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // weights -> LDS in fragment order: per output block (its weight pointer
    // uniform), all of a thread's chunks of the block loaded before any is
    // stored
    constexpr int BCH = NT * NKS * 64;            // chunks per block
    constexpr int NPT = BCH / (WAVES * 64);       // chunks per thread
    static_assert(BCH % (WAVES * 64) == 0, "whole chunks per thread");
    for (int blk = 0; blk < nblk; ++blk) {
        const T *W = reinterpret_cast<const T *>(a.out[blk].w);
        uint4 v[NPT];
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int c = threadIdx.x + k * WAVES * 64;
            const int f = c >> 6, l = c & 63;
            const int ks = f % NKS, nt = f / NKS;
            v[k] = *reinterpret_cast<const uint4 *>(W + (int64_t)(nt * 16 + (l & 15)) * E +
                                                    ks * Elem<T>::kStep + (l >> 4) * Elem<T>::kVec);
        }
#pragma unroll
        for (int k = 0; k < NPT; ++k)
            *reinterpret_cast<uint4 *>(wl + (blk * BCH + threadIdx.x + k * WAVES * 64) * 16) = v[k];
    }
    for (int blk = 0; blk < nblk; ++blk) {
        const T *bias = reinterpret_cast<const T *>(a.out[blk].b);
        for (int n = threadIdx.x; n < E; n += WAVES * 64) {
            float v = 0.f;
            if (bias) {
                if constexpr (sizeof(T) == 2)
                    v = bf2f(bias[n]);
                else
                    v = bias[n];
            }
            bl[blk * E + n] = v;
        }
    }
    __syncthreads();

    const int64_t tile_rows = (int64_t)WAVES * ROWS;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    uint4 xf[RG][NKS], xn[RG][NKS];
    auto load_x = [&](int64_t tile, uint4 (&dst)[RG][NKS]) {
        const int64_t row0 = tile * tile_rows + wid * ROWS;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int64_t r = row0 + rg * 16 + lr;
            const T *xr = reinterpret_cast<const T *>(a.x) + in_row(a, r < a.rows ? r : 0) * E +
                          lg * Elem<T>::kVec;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                dst[rg][ks] = *reinterpret_cast<const uint4 *>(xr + ks * Elem<T>::kStep);
        }
    };
    int64_t tile = blockIdx.x;
    if (tile < ntiles)
        load_x(tile, xf);
    for (; tile < ntiles; tile += gridDim.x) {
        const int64_t next = tile + gridDim.x;
        if (next < ntiles)
            load_x(next, xn);
        const int64_t row0 = tile * tile_rows + wid * ROWS;
        // (sample, token) of this lane's first stored row, once per tile
        const int cr = lane % CPR, rr = lane / CPR;
        int64_t sb0, si0;
        decompose(a, row0 + rr, sb0, si0);
        // unstaged: (sample, token) of the row each row group's lane holds
        int64_t db[RG], di[RG];
        if constexpr (!STAGE) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                decompose(a, row0 + rg * 16 + lr, db[rg], di[rg]);
        }
        for (int blk = 0; blk < nblk; ++blk) {
            const ProjOut &o = a.out[blk];
#pragma unroll 2
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc[RG];
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
                    acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const uint4 wf = *reinterpret_cast<const uint4 *>(
                        wl + (((blk * NT + nt) * NKS + ks) * 64 + lane) * 16);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg) {
                        if constexpr (sizeof(T) == 2) {
                            acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, xf[rg][ks]),
                                acc[rg], 0, 0, 0);
                        } else {
                            const float *wv = reinterpret_cast<const float *>(&wf);
                            const float *xv = reinterpret_cast<const float *>(&xf[rg][ks]);
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[rg] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[j], xv[j], acc[rg], 0, 0, 0);
                        }
                    }
                }
                // lane holds channels n = nt*16 + 4*lg + i of row (rg*16 + lr)
                const int n = nt * 16 + 4 * lg;
                const float4 b4 = *reinterpret_cast<const float4 *>(bl + blk * E + n);
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    if constexpr (STAGE) {
                        char *d = stage + (rg * 16 + lr) * PITCH + n * (int)sizeof(T);
                        uint2 pk;
                        pk.x = pack_bf16(acc[rg][0] + bv[0], acc[rg][1] + bv[1]);
                        pk.y = pack_bf16(acc[rg][2] + bv[2], acc[rg][3] + bv[3]);
                        *reinterpret_cast<uint2 *>(d) = pk;
                    } else if (row0 + rg * 16 + lr < a.rows) {
                        T *d = reinterpret_cast<T *>(o.dst) + db[rg] * o.sb + di[rg] * o.si + n;
                        *reinterpret_cast<float4 *>(d) = make_float4(
                            acc[rg][0] + bv[0], acc[rg][1] + bv[1], acc[rg][2] + bv[2], acc[rg][3] + bv[3]);
                    }
                }
            }
            if constexpr (!STAGE)
                continue;
            // a wavefront reads back only its own staged rows (LDS operations
            // of one wavefront complete in order)
            T *dst = reinterpret_cast<T *>(o.dst) + cr * (16 / (int)sizeof(T));
            int64_t sb = sb0, si = si0;
#pragma unroll
            for (int it = 0; it < ROWS / RPI; ++it) {
                const int lrow = it * RPI + rr;
                const int64_t r = row0 + lrow;
                if (r < a.rows) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(stage + lrow * PITCH + cr * 16);
                    *reinterpret_cast<uint4 *>(dst + sb * o.sb + si * o.si) = v;
                }
                advance(a, sb, si, RPI);
            }
        }
        if (next < ntiles) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) xf[rg][ks] = xn[rg][ks];
        }
    }
}

// fp32 values as the sum of three bf16 values: hi = bf16(x), mid =
// bf16(x - hi), lo = bf16(x - hi - mid). Each rounding keeps the next 8
// significant bits and the differences are exact in fp32, so hi + mid + lo
// is x itself (24 significant bits) for every x away from the bottom of the
// exponent range. Eight consecutive values become three bf16x8 operands.
__device__ inline void split3(const float (&x)[8], uint4 &h, uint4 &m, uint4 &l)
{
    float r1[8], r2[8];
    uint32_t hw[4], mw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hw[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
        r1[2 * i] = x[2 * i] - bf2f((uint16_t)(hw[i] & 0xffffu));
        r1[2 * i + 1] = x[2 * i + 1] - bf2f((uint16_t)(hw[i] >> 16));
        mw[i] = pack_bf16(r1[2 * i], r1[2 * i + 1]);
        r2[2 * i] = r1[2 * i] - bf2f((uint16_t)(mw[i] & 0xffffu));
        r2[2 * i + 1] = r1[2 * i + 1] - bf2f((uint16_t)(mw[i] >> 16));
        lw[i] = pack_bf16(r2[2 * i], r2[2 * i + 1]);
    }
    h = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    m = make_uint4(mw[0], mw[1], mw[2], mw[3]);
    l = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

// fp32 projection at embed_dim 128 on the bf16 matrix cores: x W^T with x
// and W each split into three bf16 parts (split3) and six of the nine part
// products summed in fp32 (hi hi, hi mid, mid hi, hi lo, lo hi, mid mid;
// the three left out are below 2^-23 of each product, the size of an fp32
// rounding). Per 32 multiply-adds of a lane the fp32 path issues eight
// v_mfma_f32_16x16x4f32 and this one six v_mfma_f32_16x16x32_bf16, each at
// twice the rate: 6/16 of the fp32 matrix-core time. One output block per launch: its weight parts
// fill 96 KB of LDS in fragment order (part, n-tile, k-step; lane (m, g)
// holds W[16 n-tile + m][32 k-step + 8 g .. + 7]); the workgroup's 16
// wavefronts walk tiles of 16 rows each, the next tile's x loaded ahead.
// Lane (n, g) of a wavefront loads x[row n][32 ks + 8 g .. + 7] and ends
// with output channels 16 nt + 4 g .. + 3 of row n, which it stores.
constexpr int kX3Waves = 16;
constexpr size_t kX3Lds = 3 * 8 * 4 * 1024 + 128 * 4;
__global__ void __launch_bounds__(kX3Waves * 64) proj_x3(ProjArgs a)
{
    constexpr int E = 128, NT = E / 16, NKS = E / 32;
    constexpr int PART = NT * NKS * 1024;     // bytes of one weight part
    extern __shared__ __attribute__((aligned(16))) char lds[];
    float *bl = reinterpret_cast<float *>(lds + 3 * PART);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int ln = lane & 15, lg = lane >> 4;
    const ProjOut &o = a.out[0];
    {
        const float *W = reinterpret_cast<const float *>(o.w);
        for (int f = threadIdx.x; f < NT * NKS * 64; f += kX3Waves * 64) {
            const int l = f & 63, fk = f >> 6, ks = fk % NKS, nt = fk / NKS;
            const float *wr = W + (nt * 16 + (l & 15)) * E + ks * 32 + (l >> 4) * 8;
            const float4 w0 = *reinterpret_cast<const float4 *>(wr);
            const float4 w1 = *reinterpret_cast<const float4 *>(wr + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            uint4 h, m, lo;
            split3(wv, h, m, lo);
            *reinterpret_cast<uint4 *>(lds + f * 16) = h;
            *reinterpret_cast<uint4 *>(lds + PART + f * 16) = m;
            *reinterpret_cast<uint4 *>(lds + 2 * PART + f * 16) = lo;
        }
        const float *bias = reinterpret_cast<const float *>(o.b);
        for (int n = threadIdx.x; n < E; n += kX3Waves * 64)
            bl[n] = bias ? bias[n] : 0.f;
    }
    __syncthreads();

    const int64_t tile_rows = (int64_t)kX3Waves * 16;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    uint4 xn[NKS][2];
    auto load_x = [&](int64_t tile) {
        const int64_t r = tile * tile_rows + wid * 16 + ln;
        const float *xr = reinterpret_cast<const float *>(a.x) + in_row(a, r < a.rows ? r : 0) * E +
                          lg * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            xn[ks][0] = *reinterpret_cast<const uint4 *>(xr + ks * 32);
            xn[ks][1] = *reinterpret_cast<const uint4 *>(xr + ks * 32 + 4);
        }
    };
    int64_t tile = blockIdx.x;
    if (tile < ntiles)
        load_x(tile);
    for (; tile < ntiles; tile += gridDim.x) {
        uint4 xh[NKS], xm[NKS], xl[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const float xv[8] = {__uint_as_float(xn[ks][0].x), __uint_as_float(xn[ks][0].y),
                                 __uint_as_float(xn[ks][0].z), __uint_as_float(xn[ks][0].w),
                                 __uint_as_float(xn[ks][1].x), __uint_as_float(xn[ks][1].y),
                                 __uint_as_float(xn[ks][1].z), __uint_as_float(xn[ks][1].w)};
            split3(xv, xh[ks], xm[ks], xl[ks]);
        }
        if (tile + gridDim.x < ntiles)
            load_x(tile + gridDim.x);
        const int64_t r = tile * tile_rows + wid * 16 + ln;
        int64_t db, di;
        decompose(a, r, db, di);
#pragma unroll 2
        for (int nt = 0; nt < NT; ++nt) {
            const int n = nt * 16 + 4 * lg;
            const float4 b4 = *reinterpret_cast<const float4 *>(bl + n);
            f32x4 acc = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const char *fr = lds + ((nt * NKS + ks) * 64 + lane) * 16;
                const bf16x8 wh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(fr));
                const bf16x8 wm = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(fr + PART));
                const bf16x8 wl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(fr + 2 * PART));
                const bf16x8 ph = __builtin_bit_cast(bf16x8, xh[ks]);
                const bf16x8 pm = __builtin_bit_cast(bf16x8, xm[ks]);
                const bf16x8 pl = __builtin_bit_cast(bf16x8, xl[ks]);
                // smallest products first
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wm, pm, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, ph, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, pl, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wm, ph, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, pm, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, ph, acc, 0, 0, 0);
            }
            if (r < a.rows) {
                float *d = reinterpret_cast<float *>(o.dst) + db * o.sb + di * o.si + n;
                *reinterpret_cast<float4 *>(d) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
    }
}

// Any embed_dim: one thread per (row, output channel), fp32 fused multiply-add.
template <typename T>
__global__ void __launch_bounds__(256) proj_generic(ProjArgs a, int E)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t r = idx / E;
    const int o = (int)(idx - r * E);
    if (r >= a.rows)
        return;
    const T *x = reinterpret_cast<const T *>(a.x) + in_row(a, r) * E;
    for (int blk = 0; blk < a.nblk; ++blk) {
        const ProjOut &po = a.out[blk];
        const T *w = reinterpret_cast<const T *>(po.w) + (int64_t)o * E;
        float acc = 0.f;
        for (int i = 0; i < E; ++i) {
            if constexpr (sizeof(T) == 2)
                acc = fmaf(bf2f(x[i]), bf2f(w[i]), acc);
            else
                acc = fmaf(x[i], w[i], acc);
        }
        if (po.b) {
            if constexpr (sizeof(T) == 2)
                acc += bf2f(reinterpret_cast<const T *>(po.b)[o]);
            else
                acc += reinterpret_cast<const T *>(po.b)[o];
        }
        T *d = reinterpret_cast<T *>(po.dst) + out_offset(a, po, (uint32_t)r) + o;
        if constexpr (sizeof(T) == 2)
            *d = f2bf(acc);
        else
            *d = acc;
    }
}

int cu_count()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

constexpr int kLdsBytes = 160 * 1024;

template <typename T, int K, int RG, int WAVES>
hipError_t run_mfma(const ProjArgs &a, hipStream_t s)
{
    constexpr int NKS = K / Elem<T>::kStep;
    constexpr int PITCH = K * (int)sizeof(T) + 16;
    const size_t wbytes = (size_t)a.nblk * (K / 16) * NKS * 1024 + (size_t)a.nblk * K * 4;
    const size_t lds = wbytes + (sizeof(T) == 2 ? (size_t)WAVES * RG * 16 * PITCH : 0);
    if (lds > (size_t)kLdsBytes) {
        // weights of all blocks do not fit: one launch per output block
        for (int j = 0; j < a.nblk; ++j) {
            ProjArgs one = a;
            one.nblk = 1;
            one.out[0] = a.out[j];
            hipError_t e = run_mfma<T, K, RG, WAVES>(one, s);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    const int64_t tile_rows = (int64_t)WAVES * RG * 16;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    const int per_cu = (int)(kLdsBytes / lds) < 4 ? (int)(kLdsBytes / lds) : 4;
    int64_t grid = (int64_t)cu_count() * (per_cu > 0 ? per_cu : 1);
    if (grid > ntiles)
        grid = ntiles;
    if (lds > 64 * 1024) {
        static bool raised = false;   // once per instantiation
        if (!raised) {
            hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(&proj_mfma<T, K, RG, WAVES>),
                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
            if (e != hipSuccess)
                return e;
            raised = true;
        }
    }
    hipLaunchKernelGGL((proj_mfma<T, K, RG, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64),
                       lds, s, a);
    return hipGetLastError();
}

hipError_t run_x3(const ProjArgs &a, hipStream_t s)
{
    static bool raised = false;
    if (!raised) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&proj_x3),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess)
            return e;
        raised = true;
    }
    const int64_t tile_rows = (int64_t)kX3Waves * 16;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    const int64_t grid = ntiles < cu_count() ? ntiles : cu_count();
    for (int j = 0; j < a.nblk; ++j) {   // one output block per launch
        ProjArgs one = a;
        one.nblk = 1;
        one.out[0] = a.out[j];
        hipLaunchKernelGGL(proj_x3, dim3((unsigned)grid), dim3(kX3Waves * 64), kX3Lds, s, one);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t run_generic(const ProjArgs &a, int64_t E, hipStream_t s)
{
    const int64_t n = a.rows * E;
    proj_generic<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, (int)E);
    return hipGetLastError();
}

}  // namespace

pma_status launch_proj(const ProjArgs &a, int64_t E, pma_dtype dt, hipStream_t s)
{
    if (a.rows <= 0)
        return PMA_OK;
    // The matrix-core kernels use 16-byte loads and 8/16-byte stores.
    uintptr_t bits = (uintptr_t)a.x;
    for (int j = 0; j < a.nblk; ++j)
        bits |= (uintptr_t)a.out[j].w | (uintptr_t)a.out[j].dst;
    const bool aligned = (bits & 15) == 0;
    hipError_t e;
    if (!aligned) {
        e = dt == PMA_BF16 ? run_generic<uint16_t>(a, E, s) : run_generic<float>(a, E, s);
    } else if (dt == PMA_BF16) {
        if (E == 64)   // two row groups per wavefront: 31 against 33 us for gene's k, v
            e = run_mfma<uint16_t, 64, 2, 8>(a, s);
        else if (E == 128)
            e = run_mfma<uint16_t, 128, 1, 8>(a, s);
        else
            e = run_generic<uint16_t>(a, E, s);
    } else {
        if (E == 64)
            e = run_mfma<float, 64, 1, 8>(a, s);
        else if (E == 128 && a.x3)
            e = run_x3(a, s);
        else if (E == 128 && a.rows >= (int64_t)cu_count() * 16 * 16 * 2)
            // 64 KB of weights per output block leave room for one or two
            // workgroups per CU: 16 wavefronts each keep the matrix cores busy
            // when there are enough rows for every CU
            e = run_mfma<float, 128, 1, 16>(a, s);
        else if (E == 128)
            e = run_mfma<float, 128, 1, 8>(a, s);
        else
            e = run_generic<float>(a, E, s);
    }
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
