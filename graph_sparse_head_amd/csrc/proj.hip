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

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ inline uint16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kVec = 4;    // elements per 16-byte load
    static constexpr int kStep = 16;  // k covered by one 16-byte load per lane group
};
template <> struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    static constexpr int kStep = 32;
};

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

// One wave computes RG x 16 token rows for every output channel of every
// block. Each block's tile goes through LDS so that the stores are whole
// 16-byte chunks of whole rows (the destination rows of consecutive tokens
// are far apart in the q / k / v layouts).
template <typename T, int K, int RG>
__global__ void __launch_bounds__(256) proj_mfma(ProjArgs a)
{
    constexpr int NKS = K / Elem<T>::kStep;
    constexpr int E = K;
    constexpr int ROWS = RG * 16;
    constexpr int PITCH = E * (int)sizeof(T) + 16;       // bytes per staged row
    constexpr int CPR = E * (int)sizeof(T) / 16;         // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                        // rows stored per instruction
    __shared__ __attribute__((aligned(16))) char stage_all[4][ROWS * PITCH];
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    char *stage = stage_all[wid];
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t row0 = wave * ROWS;
    if (row0 >= a.rows)
        return;
    const int lr = lane & 15, lg = lane >> 4;

    // Token-row fragments: row (row0 + rg*16 + lr), k = ks*kStep + lg*kVec ..
    uint4 xf[RG][NKS];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int64_t r = row0 + rg * 16 + lr;
        const T *xr = reinterpret_cast<const T *>(a.x) + r * E + lg * Elem<T>::kVec;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (r < a.rows)
                xf[rg][ks] = *reinterpret_cast<const uint4 *>(xr + ks * Elem<T>::kStep);
            else
                xf[rg][ks] = make_uint4(0, 0, 0, 0);
        }
    }

    for (int blk = 0; blk < a.nblk; ++blk) {
        const ProjOut &o = a.out[blk];
        const T *W = reinterpret_cast<const T *>(o.w);
        const T *bias = reinterpret_cast<const T *>(o.b);
        for (int nt = 0; nt < E / 16; ++nt) {
            uint4 wf[NKS];
            const T *wr = W + (int64_t)(nt * 16 + lr) * E + lg * Elem<T>::kVec;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                wf[ks] = *reinterpret_cast<const uint4 *>(wr + ks * Elem<T>::kStep);
            f32x4 acc[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    if constexpr (sizeof(T) == 2) {
                        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wf[ks]), __builtin_bit_cast(bf16x8, xf[rg][ks]),
                            acc[rg], 0, 0, 0);
                    } else {
                        const float *wv = reinterpret_cast<const float *>(&wf[ks]);
                        const float *xv = reinterpret_cast<const float *>(&xf[rg][ks]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[rg] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[j], xv[j], acc[rg], 0, 0, 0);
                    }
                }
            }
            // lane holds channels n = nt*16 + 4*lg + i of token row (rg*16 + lr)
            const int n = nt * 16 + 4 * lg;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (sizeof(T) == 2)
                        bv[i] = bf2f(bias[n + i]);
                    else
                        bv[i] = bias[n + i];
                }
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                char *d = stage + (rg * 16 + lr) * PITCH + n * (int)sizeof(T);
                if constexpr (sizeof(T) == 2) {
                    uint2 pk;
                    pk.x = (uint32_t)f2bf(acc[rg][0] + bv[0]) | ((uint32_t)f2bf(acc[rg][1] + bv[1]) << 16);
                    pk.y = (uint32_t)f2bf(acc[rg][2] + bv[2]) | ((uint32_t)f2bf(acc[rg][3] + bv[3]) << 16);
                    *reinterpret_cast<uint2 *>(d) = pk;
                } else {
                    *reinterpret_cast<float4 *>(d) = make_float4(
                        acc[rg][0] + bv[0], acc[rg][1] + bv[1], acc[rg][2] + bv[2], acc[rg][3] + bv[3]);
                }
            }
        }
        // the wave reads back its own staged rows: no cross-wave sharing
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        T *dst = reinterpret_cast<T *>(o.dst);
        const int cr = lane % CPR, rr = lane / CPR;
#pragma unroll
        for (int it = 0; it < ROWS / RPI; ++it) {
            const int lrow = it * RPI + rr;
            const int64_t r = row0 + lrow;
            if (r < a.rows) {
                const uint4 v = *reinterpret_cast<const uint4 *>(stage + lrow * PITCH + cr * 16);
                T *dp = dst + out_offset(a, o, (uint32_t)r) + cr * (16 / (int)sizeof(T));
                *reinterpret_cast<uint4 *>(dp) = v;
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    const T *x = reinterpret_cast<const T *>(a.x) + r * E;
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

template <typename T, int K, int RG>
hipError_t run_mfma(const ProjArgs &a, hipStream_t s)
{
    const int64_t waves = (a.rows + RG * 16 - 1) / (RG * 16);
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    proj_mfma<T, K, RG><<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
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
        if (E == 64)
            e = run_mfma<uint16_t, 64, 4>(a, s);
        else if (E == 128)
            e = run_mfma<uint16_t, 128, 2>(a, s);
        else
            e = run_generic<uint16_t>(a, E, s);
    } else {
        if (E == 64)
            e = run_mfma<float, 64, 2>(a, s);
        else if (E == 128)
            e = run_mfma<float, 128, 1>(a, s);
        else
            e = run_generic<float>(a, E, s);
    }
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
