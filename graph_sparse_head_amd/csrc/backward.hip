// Backward pass of packed multi-head attention over live edges (kpnn2
// PackedMultiheadAttention page, "Notes" steps 1-5, differentiated; the
// page's layer trains with torch autograd, this library computes the same
// gradients directly).
//
// With mixed_h[t] = sum_e p_e v_h[s_e], p the softmax of the scores
// z_e = dot(q_h[t], k_h[s_e]) / sqrt(d) over the edges into t, and dm = the
// gradient reaching mixed (dO Wo), per (sample, target, head):
//   dp_e = dot(dm_h[t], v_h[s_e]),  D = dot(dm_h[t], mixed_h[t]) = sum_e p_e dp_e,
//   dz_e = p_e (dp_e - D),
//   dq_h[t] = sum_e dz_e k_h[s_e] / sqrt(d),
//   dk_h[s] = sum over edges e out of s of dz_e q_h[t_e] / sqrt(d),
//   dv_h[s] = sum over edges e out of s of p_e dm_h[t_e].
// The weights p_e are recomputed from the forward's saved scores' (max, sum)
// per (target, sample, head), in base 2 as the forward computed them. A
// first pass walks each target's edges (dq, and p_e, dz_e per edge); a
// second walks each source's edges through the source-major index (dk, dv),
// so neither needs atomics. Masked keys have p = dz = 0.
//
// Layouts (batch-first): q, mixed (B, L, E) and k, v (B, S, E) in the plan's
// dtype; dm, dq (B, L, E) and dk, dv (B, S, E) fp32; ml [L][B][H][2];
// P and DZ [nnz][B][H] by target-grouped position.
#include "pma_internal.h"

namespace pma {
namespace {

template <typename T> __device__ inline float ld(const T *p);
template <> __device__ inline float ld<float>(const float *p) { return *p; }
template <> __device__ inline float ld<uint16_t>(const uint16_t *p)
{
    return __uint_as_float((uint32_t)*p << 16);
}

// One thread per (target, sample, head); DD = head size when fixed at
// compile time (registers), 0 for any head size up to 64.
template <typename T, int DD>
__global__ void __launch_bounds__(256)
bwd_target(const BwdArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.L * a.B * a.H;
    if (i >= n)
        return;
    const int h = (int)(i % a.H);
    const int64_t bt = i / a.H;
    const int b = (int)(bt % a.B);
    const int t = (int)(bt / a.B);
    const int d = DD > 0 ? DD : a.E / a.H;
    const T *q = reinterpret_cast<const T *>(a.q) + ((int64_t)b * a.L + t) * a.E + h * d;
    const T *mx = reinterpret_cast<const T *>(a.mixed) + ((int64_t)b * a.L + t) * a.E + h * d;
    const float *dm = a.dm + ((int64_t)b * a.L + t) * a.E + h * d;
    const float2 ml = *reinterpret_cast<const float2 *>(a.ml + (((int64_t)t * a.B + b) * a.H + h) * 2);
    float D = 0.f;
    for (int c = 0; c < d; ++c)
        D = fmaf(dm[c], ld(mx + c), D);
    float dq[DD > 0 ? DD : 64];
#pragma unroll
    for (int c = 0; c < (DD > 0 ? DD : 64); ++c)
        dq[c] = 0.f;
    const int beg = a.row_ptr[t], end = a.row_ptr[t + 1];
    const T *K = reinterpret_cast<const T *>(a.k);
    const T *V = reinterpret_cast<const T *>(a.v);
    for (int p = beg; p < end; ++p) {
        const int s = a.csr_src[p];
        float pe = 0.f, dz = 0.f;
        const bool masked =
            a.kpm_bits && ((a.kpm_bits[(int64_t)s * a.kpm_words + (b >> 6)] >> (b & 63)) & 1u);
        if (!masked && ml.y > 0.f) {
            const T *kr = K + ((int64_t)b * a.S + s) * a.E + h * d;
            const T *vr = V + ((int64_t)b * a.S + s) * a.E + h * d;
            float z = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < (DD > 0 ? DD : 64); ++c) {
                if (DD == 0 && c >= d)
                    break;
                z = fmaf(ld(q + c), ld(kr + c), z);
                dp = fmaf(dm[c], ld(vr + c), dp);
            }
            pe = __builtin_amdgcn_exp2f(z * a.scale_log2 - ml.x) / ml.y;
            dz = pe * (dp - D);
#pragma unroll
            for (int c = 0; c < (DD > 0 ? DD : 64); ++c) {
                if (DD == 0 && c >= d)
                    break;
                dq[c] = fmaf(dz, ld(kr + c), dq[c]);
            }
        }
        const int64_t o = ((int64_t)p * a.B + b) * a.H + h;
        a.P[o] = pe;
        a.DZ[o] = dz;
    }
    float *out = a.dq + ((int64_t)b * a.L + t) * a.E + h * d;
#pragma unroll
    for (int c = 0; c < (DD > 0 ? DD : 64); ++c) {
        if (DD == 0 && c >= d)
            break;
        out[c] = dq[c] * a.inv_sqrt_d;
    }
}

// One thread per (source, sample, channel).
template <typename T>
__global__ void __launch_bounds__(256)
bwd_source(const BwdArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.S * a.B * a.E;
    if (i >= n)
        return;
    const int c = (int)(i % a.E);
    const int64_t bs = i / a.E;
    const int b = (int)(bs % a.B);
    const int s = (int)(bs / a.B);
    const int h = c / (a.E / a.H);
    const T *Q = reinterpret_cast<const T *>(a.q);
    float dk = 0.f, dv = 0.f;
    for (int j = a.csc_ptr[s]; j < a.csc_ptr[s + 1]; ++j) {
        const int t = a.csc_tgt[j];
        const int64_t o = ((int64_t)a.csc_pos[j] * a.B + b) * a.H + h;
        const int64_t r = ((int64_t)b * a.L + t) * a.E + c;
        dk = fmaf(a.DZ[o], ld(Q + r), dk);
        dv = fmaf(a.P[o], a.dm[r], dv);
    }
    const int64_t w = ((int64_t)b * a.S + s) * a.E + c;
    a.dk[w] = dk * a.inv_sqrt_d;
    a.dv[w] = dv;
}

template <typename T>
__global__ void to_f32_kernel(const T *x, float *y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        y[i] = ld(x + i);
}

__global__ void f32_to_bf16_kernel(const float *x, uint16_t *y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        // round to nearest even
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        typedef __attribute__((ext_vector_type(2))) float f32x2;
        const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[i], 0.f}, bf16x2));
        y[i] = (uint16_t)(w & 0xffffu);
    }
}

// Column sums of a (rows, E) fp32 matrix: one block per column.
__global__ void __launch_bounds__(256) colsum_kernel(const float *g, int64_t rows, int E, float *out)
{
    const int c = blockIdx.x;
    float acc = 0.f;
    for (int64_t r = threadIdx.x; r < rows; r += blockDim.x)
        acc += g[r * E + c];
    __shared__ float red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[c] = red[0];
}

inline unsigned grid(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

pma_status launch_bwd_edges(const BwdArgs &a, pma_dtype dt, hipStream_t s)
{
    if (a.E / a.H > 64)
        return PMA_E_UNSUPPORTED;
    const int64_t nt = (int64_t)a.L * a.B * a.H, ns = (int64_t)a.S * a.B * a.E;
    const int d = (int)(a.E / a.H);
    auto target = [&](auto tag) {
        using T = decltype(tag);
        switch (d) {
        case 4: bwd_target<T, 4><<<grid(nt), 256, 0, s>>>(a); break;
        case 8: bwd_target<T, 8><<<grid(nt), 256, 0, s>>>(a); break;
        case 16: bwd_target<T, 16><<<grid(nt), 256, 0, s>>>(a); break;
        case 32: bwd_target<T, 32><<<grid(nt), 256, 0, s>>>(a); break;
        default: bwd_target<T, 0><<<grid(nt), 256, 0, s>>>(a); break;
        }
        bwd_source<T><<<grid(ns), 256, 0, s>>>(a);
    };
    if (dt == PMA_BF16)
        target(uint16_t{});
    else
        target(float{});
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status to_f32(const void *x, pma_dtype dt, float *y, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return PMA_OK;
    if (dt == PMA_BF16)
        to_f32_kernel<uint16_t><<<grid(n), 256, 0, s>>>(reinterpret_cast<const uint16_t *>(x), y, n);
    else
        return hipMemcpyAsync(y, x, n * sizeof(float), hipMemcpyDeviceToDevice, s) == hipSuccess
                   ? PMA_OK
                   : PMA_E_DEVICE;
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status from_f32(const float *x, pma_dtype dt, void *y, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return PMA_OK;
    if (dt == PMA_BF16)
        f32_to_bf16_kernel<<<grid(n), 256, 0, s>>>(x, reinterpret_cast<uint16_t *>(y), n);
    else
        return hipMemcpyAsync(y, x, n * sizeof(float), hipMemcpyDeviceToDevice, s) == hipSuccess
                   ? PMA_OK
                   : PMA_E_DEVICE;
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status colsum(const float *g, int64_t rows, int E, float *out, hipStream_t s)
{
    colsum_kernel<<<E, 256, 0, s>>>(g, rows, E, out);
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
