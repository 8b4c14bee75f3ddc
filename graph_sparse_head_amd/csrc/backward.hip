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
// The weights p_e are recomputed from the forward's saved (max, sum) per
// (target, sample, head), in base 2 as the forward computed them. A first
// pass walks each target's edges (dq); a second walks each source's edges
// through the source-major index (dk, dv), so neither needs atomics. The
// second needs p_e and dz_e again: with 16-byte lanes it recomputes them from
// the target's q and dm rows and a per-(target, sample, head) pair
// (m + log2 l, D) the first pass leaves; the per-channel path stores them per
// edge instead. Long edge lists are cut into pieces whose partial sums a
// merge adds up in a fixed order. Masked keys have p = dz = 0.
//
// The linear maps around it: for y = x W^T + b, dx = dy W (rowmm below) and
// dW = dy^T x, db = column sums of dy (wgrad below), both on the matrix cores.
//
// Layouts (batch-first, plan dtype T unless noted): q, mixed, dm, dq (B, L, E);
// k, v, dk, dv (B, S, E); ml and (m + log2 l, D) [L][B][H][2] fp32; on the
// per-channel path (p, dz) pairs [nnz][B][H] by target-grouped position (bf16
// pairs for bf16 plans, fp32 pairs otherwise). Gradient tensors are stored in
// T and accumulated in fp32.
#include "pma_internal.h"

#include <algorithm>
#include <type_traits>

namespace pma {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ inline float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// two fp32 -> packed bf16, round to nearest even
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ inline uint16_t f2bf(float f) { return (uint16_t)(pack_bf16(f, 0.f) & 0xffffu); }

template <typename T> __device__ inline float ld(const T *p);
template <> __device__ inline float ld<float>(const float *p) { return *p; }
template <> __device__ inline float ld<uint16_t>(const uint16_t *p) { return bf2f(*p); }
template <typename T> __device__ inline void st(T *p, float x);
template <> __device__ inline void st<float>(float *p, float x) { *p = x; }
template <> __device__ inline void st<uint16_t>(uint16_t *p, float x) { *p = f2bf(x); }

// 16 bytes of T widened to fp32 (4 floats or 8 bf16), and back
template <typename T> struct Vec {
    static constexpr int N = 16 / (int)sizeof(T);
};
// 16-byte loads and stores past the caches (rows read or written once)
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_nt;
__device__ inline uint4 ld16_nt(const void *p)
{
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename T>
__device__ inline void store_vec(T *p, const float (&f)[Vec<T>::N], bool nt = false)
{
    uint4 u;
    if constexpr (sizeof(T) == 4) {
        u = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                       __float_as_uint(f[3]));
    } else {
        u = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                       pack_bf16(f[6], f[7]));
    }
    if (nt)
        __builtin_nontemporal_store(u32x4_nt{u.x, u.y, u.z, u.w}, reinterpret_cast<u32x4_nt *>(p));
    else
        *reinterpret_cast<uint4 *>(p) = u;
}
template <int N> __device__ inline void store_f32(float *p, const float (&f)[N])
{
#pragma unroll
    for (int i = 0; i < N; i += 4)
        *reinterpret_cast<float4 *>(p + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
}

template <int CTRL> __device__ inline float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of G lanes (all of them active); every lane of
// the group ends with the same bits.
template <int G> __device__ inline float group_sum(float x)
{
    if constexpr (G >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (G >= 16) x += dpp<0x140>(x); // row_mirror
    return x;
}

__device__ inline bool masked(const BwdArgs &a, int s, int b)
{
    return a.kpm_bits &&
           ((a.kpm_bits[(int64_t)s * a.kpm_words + (b >> 6)] >> (b & 63)) & 1u);
}

// Per-channel path, per (edge, sample, head): the weight p and the score
// gradient dz, stored together: a bf16 pair (round to nearest even) for bf16
// plans, an fp32 pair otherwise.
template <typename T> __device__ inline void put_pz(void *pz, int64_t o, float p, float dz)
{
    if constexpr (sizeof(T) == 2)
        reinterpret_cast<uint32_t *>(pz)[o] = pack_bf16(p, dz);
    else
        reinterpret_cast<float2 *>(pz)[o] = make_float2(p, dz);
}
template <typename T> __device__ inline float2 get_pz(const void *pz, int64_t o)
{
    if constexpr (sizeof(T) == 2) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(pz)[o];
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    } else {
        return reinterpret_cast<const float2 *>(pz)[o];
    }
}

constexpr int kU = 4;   // edges whose rows are loaded together

template <typename T> __device__ inline void widen(const uint4 &u, float (&f)[Vec<T>::N])
{
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
__device__ inline uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// ---- edge passes, 16-byte lanes -----------------------------------------
// Thread = (piece, sample, 16-byte chunk of the row), chunks fastest; LPH
// chunks make one head. With UNI the host has checked that a piece's lanes
// fill whole wavefronts, so the piece and its edge indices are wavefront-
// uniform and go through scalar loads. Index arrays carry kSrcPad zero
// entries past their end, so kU entries are read at a time without clamping
// (entry 0 is a valid row); the next kU edges' rows are in flight while the
// current ones are used.

// CM (UNI only): the mask comes as one uniform word per CSR position
// (kpm_csr); otherwise each lane looks its bit up by source.
// bf16 plans keep q and dm packed and form the dot products with v_dot2.
// PF: the next kU edges' rows are requested before the current ones are
// used (twice the row registers); otherwise each step loads, then uses (at
// most 80 registers: 6 wavefronts per SIMD).
template <typename T, int LPH, bool UNI, bool CM = false, bool PF = true>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PF ? 1 : 6)))
bwd_target_fast(const BwdArgs a)
{
    constexpr int VEC = Vec<T>::N;
    constexpr bool BF = sizeof(T) == 2;
    const int CPR = a.E / VEC;
    int64_t task;
    int b, c;
    if (UNI && a.t_order != 0) {
        // one wavefront per (piece, sample group): lane = sample * CPR + chunk
        int64_t i;
        int g;
        if (a.t_order == 1) {   // workgroups dealt round-robin to the 8 XCDs
            const int x = blockIdx.x & 7;
            g = x % a.t_groups;
            i = ((int64_t)(blockIdx.x >> 3) * (8 / a.t_groups) + x / a.t_groups) * blockDim.x +
                threadIdx.x;
        } else {
            const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
            g = (int)(j / a.t_gthreads);
            i = j - g * a.t_gthreads;
        }
        task = __builtin_amdgcn_readfirstlane((int)(i >> 6));
        // lane l of group g is chunk (64 g + l) of the piece's B * CPR chunks
        // (CPR need not divide 64)
        const int cg = g * 64 + (threadIdx.x & 63);
        b = cg / CPR;
        c = cg - b * CPR;
    } else {
        const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        const int64_t gb = idx / CPR;
        c = (int)(idx - gb * CPR);
        task = gb / a.B;
        b = (int)(gb - task * a.B);
        if (UNI)
            task = __builtin_amdgcn_readfirstlane((int)task);
    }
    if (task >= a.n_ttasks)
        return;
    const int t = a.t_target[task], beg = a.t_begin[task], end = a.t_end[task];
    const int slot = a.t_slot[task];
    const int h = c / LPH;
    const int64_t row = ((int64_t)b * a.L + t) * a.E + c * VEC;
    const T *qp = reinterpret_cast<const T *>(a.q) + row, *dmp = reinterpret_cast<const T *>(a.dm) + row;
    const uint4 qw = (a.nt & 2) ? ld16_nt(qp) : ld16(qp);
    const uint4 dmw = (a.nt & 2) ? ld16_nt(dmp) : ld16(dmp);
    float qv[VEC], dmv[VEC];
    widen<T>(qw, qv);
    widen<T>(dmw, dmv);
    float D = 0.f;
    {
        float mx[VEC];
        const T *mp = reinterpret_cast<const T *>(a.mixed) + row;
        widen<T>((a.nt & 1) ? ld16_nt(mp) : ld16(mp), mx);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            D = fmaf(dmv[i], mx[i], D);
    }
    D = group_sum<LPH>(D);
    const float2 ml =
        *reinterpret_cast<const float2 *>(a.ml + (((int64_t)t * a.B + b) * a.H + h) * 2);
    const bool lead = (c & (LPH - 1)) == 0;
    // For the source pass, which recomputes each edge's weight and score
    // gradient: m' = m + log2(l) (weight = exp2(z - m'); +inf when the
    // target has no live edge, so every weight is 0) and D. Every piece of a
    // split target writes the same values.
    if (lead) {
        const float mq = ml.y > 0.f ? ml.x + __builtin_amdgcn_logf(ml.y) : INFINITY;
        *reinterpret_cast<float2 *>(a.mD + (((int64_t)t * a.B + b) * a.H + h) * 2) = make_float2(mq, D);
    }
    const T *Kb = reinterpret_cast<const T *>(a.k) + (int64_t)b * a.Skv * a.E + c * VEC;
    const T *Vb = reinterpret_cast<const T *>(a.v) + (int64_t)b * a.Skv * a.E + c * VEC;
    float dq[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        dq[i] = 0.f;
    // Mask: with whole wavefronts per piece whose samples lie in one 32-sample
    // word (the host's choice of CM), one 32-bit word per CSR position
    // (uniform: a scalar load) holds the bits of the wavefront's samples;
    // otherwise each lane looks up its sample's bit by source.
    static_assert(!CM || UNI, "uniform mask words need whole wavefronts per piece");
    const uint32_t kw = CM ? (uint32_t)__builtin_amdgcn_readfirstlane(b) >> 5 : 0u;
    int s[kU], sn[kU];   // mask words (csr_mask) or sources; rows come through kv_src
    uint4 kr[kU], vr[kU], kn[kU], vn[kU];
    auto fetch = [&](int p0, int (&ss)[kU], uint4 (&kq)[kU], uint4 (&vq)[kU]) {
        int r[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if constexpr (CM)
                ss[u] = (int)a.kpm_csr[(uint32_t)(p0 + u) * (uint32_t)a.kpm_w32 + kw];
            else
                ss[u] = a.csr_src[p0 + u];
            r[u] = a.kv_src[p0 + u];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            kq[u] = ld16(Kb + (int64_t)r[u] * a.E);
            vq[u] = ld16(Vb + (int64_t)r[u] * a.E);
        }
    };
    if (PF && beg < end)
        fetch(beg, s, kr, vr);
    for (int p0 = beg; p0 < end; p0 += kU) {
        const bool more = PF && p0 + kU < end;
        if constexpr (PF) {
            if (more)
                fetch(p0 + kU, sn, kn, vn);
        } else {
            fetch(p0, s, kr, vr);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float kk[VEC];
            widen<T>(kr[u], kk);
            float z = 0.f, dp = 0.f;
            if constexpr (BF) {
                typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
                const uint32_t qa[4] = {qw.x, qw.y, qw.z, qw.w}, ma[4] = {dmw.x, dmw.y, dmw.z, dmw.w};
                const uint32_t ka[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
                const uint32_t va[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qa[w]),
                                                        __builtin_bit_cast(bf16x2_t, ka[w]), z, false);
                    dp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ma[w]),
                                                         __builtin_bit_cast(bf16x2_t, va[w]), dp, false);
                }
            } else {
                float vv[VEC];
                widen<T>(vr[u], vv);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    z = fmaf(qv[i], kk[i], z);
                    dp = fmaf(dmv[i], vv[i], dp);
                }
            }
            z = group_sum<LPH>(z);
            dp = group_sum<LPH>(dp);
            const int p = p0 + u;
            if (p < end) {
                float pe = 0.f, dz = 0.f;
                bool off;
                if constexpr (CM)
                    off = (((uint32_t)s[u] >> (b & 31)) & 1u) != 0;
                else
                    off = masked(a, s[u], b);
                if (ml.y > 0.f && !off) {
                    pe = __builtin_amdgcn_exp2f(z * a.scale_log2 - ml.x) / ml.y;
                    dz = pe * (dp - D);
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    dq[i] = fmaf(dz, kk[i], dq[i]);
            }
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                s[u] = sn[u];
                kr[u] = kn[u];
                vr[u] = vn[u];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        dq[i] *= a.inv_sqrt_d;
    if (slot < 0)
        store_vec(reinterpret_cast<T *>(a.dq) + row, dq, (a.nt & 8) != 0);
    else
        store_f32(a.part_q + ((int64_t)slot * a.B + b) * a.E + c * VEC, dq);
}

// With UNI and bands the pieces run band by band on fixed XCDs: workgroups are dealt to
// the 8 XCDs round-robin, so workgroup i serves band i mod 8, and the pieces
// of one band (sorted by target) gather their target rows through one L2.
template <typename T, int LPH, bool UNI>
__global__ void __launch_bounds__(256) bwd_source_fast(const BwdArgs a)
{
    constexpr int VEC = Vec<T>::N;
    const int CPR = a.E / VEC;
    int64_t idx, base = 0;
    if (UNI && a.banded) {
        const int band = blockIdx.x % kBands;
        base = a.s_band_off[band];
        idx = (int64_t)(blockIdx.x / kBands) * blockDim.x + threadIdx.x;
        if (idx >= (a.s_band_off[band + 1] - base) * a.B * CPR)
            return;   // whole wavefront (a piece's threads fill wavefronts)
    } else {
        idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    }
    int64_t task;
    int b, c;
    if (UNI && a.banded && a.s_order == 2) {
        // sample groups one after another within each band: the band's
        // wavefronts for group 0 first, then group 1, ..., so that the target
        // rows in flight belong to one group (lane l of group g is chunk
        // 64 g + l of the piece's B * CPR chunks)
        const int64_t nb = a.s_band_off[blockIdx.x % kBands + 1] - base;   // pieces in the band
        const int64_t g = idx / (nb * 64), rem = idx - g * nb * 64;
        task = base + rem / 64;
        const int cg = (int)(g * 64 + (rem & 63));
        b = cg / CPR;
        c = cg - b * CPR;
    } else {
        const int64_t gb = idx / CPR;
        c = (int)(idx - gb * CPR);
        task = base + gb / a.B;
        b = (int)(gb - (task - base) * a.B);
    }
    if (UNI)
        task = __builtin_amdgcn_readfirstlane((int)task);
    if (task >= a.n_stasks)
        return;
    const int s = a.s_source[task], beg = a.s_begin[task], end = a.s_end[task];
    const int slot = a.s_slot[task];
    const int h = c / LPH;
    constexpr bool BF = sizeof(T) == 2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const T *Qb = reinterpret_cast<const T *>(a.q) + (int64_t)b * a.L * a.E + c * VEC;
    const T *Mb = reinterpret_cast<const T *>(a.dm) + (int64_t)b * a.L * a.E + c * VEC;
    const float *MD = a.mD + (int64_t)b * a.H * 2 + h * 2;   // (m', D) of (t, b, h) at + t B H 2
    float dk[VEC], dv[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        dk[i] = dv[i] = 0.f;
    // The source's own key and value chunks (its saved row through the
    // compact row index of any of its edges); a key masked for this sample
    // leaves every one of its edges out (weight and score gradient 0).
    const bool live = beg < end && !masked(a, s, b);
    uint4 kw = make_uint4(0, 0, 0, 0), vw = kw;
    if (live) {
        const int r = a.kv_src[a.csc_pos[beg]];
        const T *kp = reinterpret_cast<const T *>(a.k) + ((int64_t)b * a.Skv + r) * a.E + c * VEC;
        const T *vp = reinterpret_cast<const T *>(a.v) + ((int64_t)b * a.Skv + r) * a.E + c * VEC;
        kw = (a.nt & 4) ? ld16_nt(kp) : ld16(kp);
        vw = (a.nt & 4) ? ld16_nt(vp) : ld16(vp);
    }
    float kf[BF ? 1 : VEC], vf[BF ? 1 : VEC];
    if constexpr (!BF) {
        widen<T>(kw, kf);
        widen<T>(vw, vf);
    }
    float2 md[kU], mdn[kU];
    uint4 qr[kU], mr[kU], qn[kU], mn[kU];
    auto fetch = [&](int j0, float2 (&dd)[kU], uint4 (&qq)[kU], uint4 (&mm)[kU]) {
        int t[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) t[u] = a.csc_tgt[j0 + u];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            qq[u] = ld16(Qb + (int64_t)t[u] * a.E);
            mm[u] = ld16(Mb + (int64_t)t[u] * a.E);
            dd[u] = *reinterpret_cast<const float2 *>(MD + (int64_t)t[u] * a.B * a.H * 2);
        }
    };
    // per edge: z = q_t . k_s and dp = dm_t . v_s over the head, the weight
    // p = exp2(z log2(e)/sqrt(d) - m') and dz = p (dp - D), as the target
    // pass computed them; then dk += dz q_t, dv += p dm_t
    auto batch = [&](int j0, auto full) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float z = 0.f, dp = 0.f;
            if constexpr (BF) {
                const uint32_t qa[4] = {qr[u].x, qr[u].y, qr[u].z, qr[u].w};
                const uint32_t ma[4] = {mr[u].x, mr[u].y, mr[u].z, mr[u].w};
                const uint32_t ka[4] = {kw.x, kw.y, kw.z, kw.w};
                const uint32_t va[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qa[w]),
                                                        __builtin_bit_cast(bf16x2_t, ka[w]), z, false);
                    dp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ma[w]),
                                                         __builtin_bit_cast(bf16x2_t, va[w]), dp, false);
                }
            } else {
                float qq[VEC], mm[VEC];
                widen<T>(qr[u], qq);
                widen<T>(mr[u], mm);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    z = fmaf(qq[i], kf[i], z);
                    dp = fmaf(mm[i], vf[i], dp);
                }
            }
            z = group_sum<LPH>(z);
            dp = group_sum<LPH>(dp);
            if (decltype(full)::value || j0 + u < end) {
                const float pu = live ? __builtin_amdgcn_exp2f(z * a.scale_log2 - md[u].x) : 0.f;
                const float du = pu * (dp - md[u].y);
                float qq[VEC], mm[VEC];
                widen<T>(qr[u], qq);
                widen<T>(mr[u], mm);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    dk[i] = fmaf(du, qq[i], dk[i]);
                    dv[i] = fmaf(pu, mm[i], dv[i]);
                }
            }
        }
    };
    if (live) {
        // as in the target pass: the successor is fetched first, the last
        // batch runs after the loop
        fetch(beg, md, qr, mr);
        int j0 = beg;
        for (; j0 + kU < end; j0 += kU) {
            fetch(j0 + kU, mdn, qn, mn);
            batch(j0, std::true_type{});
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                md[u] = mdn[u];
                qr[u] = qn[u];
                mr[u] = mn[u];
            }
        }
        batch(j0, std::false_type{});
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        dk[i] *= a.inv_sqrt_d;
    if (slot < 0) {
        const int64_t row = ((int64_t)b * a.S + s) * a.E + c * VEC;
        store_vec(reinterpret_cast<T *>(a.dk) + row, dk, (a.nt & 8) != 0);
        store_vec(reinterpret_cast<T *>(a.dv) + row, dv, (a.nt & 8) != 0);
    } else {
        float *d = a.part_kv + ((int64_t)slot * a.B + b) * 2 * a.E + c * VEC;
        store_f32(d, dk);
        store_f32(d + a.E, dv);
    }
}

// Sums the pieces of split targets (dq) / split sources (dk, dv): G lanes
// per (split, sample, 16-byte chunk).
template <typename T, int G>
__global__ void __launch_bounds__(256) bwd_merge_fast(const BwdArgs a, int sources)
{
    // G adjacent lanes serve one (split row, sample, 16-byte chunk): lane g
    // adds slots g, g + G, g + 2G, ... in slot order, kM of them in flight,
    // and the G partial sums meet in a fixed butterfly (deterministic; long
    // rows such as hub sources cut into hundreds of pieces no longer add
    // their slots one round trip at a time).
    constexpr int VEC = Vec<T>::N;
    const int CPR = a.E / VEC;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int g = (int)(idx & (G - 1));
    const int64_t gi = idx / G;
    const int64_t gb = gi / CPR;
    const int c = (int)(gi - gb * CPR);
    const int64_t i = gb / a.B;
    const int b = (int)(gb - i * a.B);
    if (i >= (sources ? a.n_ssplit : a.n_tsplit))
        return;   // (the whole group of G lanes)
    const int row_id = sources ? a.ss_source[i] : a.ts_target[i];
    const int slot0 = sources ? a.ss_slot0[i] : a.ts_slot0[i];
    const int count = sources ? a.ss_count[i] : a.ts_count[i];
    const int nout = sources ? 2 : 1;
    const int width = nout * a.E;
    const float *part = sources ? a.part_kv : a.part_q;
    constexpr int kM = 4;
    float acc[2][VEC];
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            acc[o][j] = 0.f;
    const float *base = part + ((int64_t)slot0 * a.B + b) * width + c * VEC;
    const int64_t sstride = (int64_t)a.B * width;
    for (int k0 = g; k0 < count; k0 += G * kM) {
        float4 v[kM][2][VEC / 4];
#pragma unroll
        for (int u = 0; u < kM; ++u) {
            if (k0 + u * G < count) {
#pragma unroll
                for (int o = 0; o < 2; ++o)
                    if (o < nout)
#pragma unroll
                        for (int j = 0; j < VEC / 4; ++j)
                            v[u][o][j] = *reinterpret_cast<const float4 *>(
                                base + (k0 + u * G) * sstride + o * a.E + 4 * j);
            }
        }
#pragma unroll
        for (int u = 0; u < kM; ++u) {
            if (k0 + u * G < count) {
#pragma unroll
                for (int o = 0; o < 2; ++o)
                    if (o < nout)
#pragma unroll
                        for (int j = 0; j < VEC / 4; ++j) {
                            acc[o][4 * j] += v[u][o][j].x;
                            acc[o][4 * j + 1] += v[u][o][j].y;
                            acc[o][4 * j + 2] += v[u][o][j].z;
                            acc[o][4 * j + 3] += v[u][o][j].w;
                        }
            }
        }
    }
    if constexpr (G > 1) {
#pragma unroll
        for (int off = 1; off < G; off <<= 1)
#pragma unroll
            for (int o = 0; o < 2; ++o)
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    acc[o][j] += __shfl_xor(acc[o][j], off, 64);
        if (g != 0)
            return;
    }
    for (int o = 0; o < nout; ++o) {
        T *dst = sources ? reinterpret_cast<T *>(o == 0 ? a.dk : a.dv) +
                               ((int64_t)b * a.S + row_id) * a.E
                         : reinterpret_cast<T *>(a.dq) + ((int64_t)b * a.L + row_id) * a.E;
        store_vec(dst + c * VEC, acc[o]);
    }
}

// ---- edge passes, any head size up to 64 ---------------------------------

// One thread per (target, sample, head), whole edge list.
template <typename T>
__global__ void __launch_bounds__(256) bwd_target_generic(const BwdArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.L * a.B * a.H;
    if (i >= n)
        return;
    const int h = (int)(i % a.H);
    const int64_t bt = i / a.H;
    const int b = (int)(bt % a.B);
    const int t = (int)(bt / a.B);
    const int d = a.E / a.H;
    const int64_t row = ((int64_t)b * a.L + t) * a.E + h * d;
    const T *q = reinterpret_cast<const T *>(a.q) + row;
    const T *mx = reinterpret_cast<const T *>(a.mixed) + row;
    const T *dm = reinterpret_cast<const T *>(a.dm) + row;
    const float2 ml =
        *reinterpret_cast<const float2 *>(a.ml + (((int64_t)t * a.B + b) * a.H + h) * 2);
    float D = 0.f;
    for (int c = 0; c < d; ++c)
        D = fmaf(ld(dm + c), ld(mx + c), D);
    float dq[64];
    for (int c = 0; c < 64; ++c)
        dq[c] = 0.f;
    const T *K = reinterpret_cast<const T *>(a.k);
    const T *V = reinterpret_cast<const T *>(a.v);
    for (int p = a.row_ptr[t]; p < a.row_ptr[t + 1]; ++p) {
        const int s = a.csr_src[p];
        float pe = 0.f, dz = 0.f;
        if (ml.y > 0.f && !masked(a, s, b)) {
            const int64_t kvr = (int64_t)b * a.Skv + a.kv_src[p];
            const T *kr = K + kvr * a.E + h * d;
            const T *vr = V + kvr * a.E + h * d;
            float z = 0.f, dp = 0.f;
            for (int c = 0; c < d; ++c) {
                z = fmaf(ld(q + c), ld(kr + c), z);
                dp = fmaf(ld(dm + c), ld(vr + c), dp);
            }
            pe = __builtin_amdgcn_exp2f(z * a.scale_log2 - ml.x) / ml.y;
            dz = pe * (dp - D);
            for (int c = 0; c < 64; ++c) {
                if (c >= d)
                    break;
                dq[c] = fmaf(dz, ld(kr + c), dq[c]);
            }
        }
        const int64_t o = ((int64_t)p * a.B + b) * a.H + h;
        put_pz<T>(a.PZ, o, pe, dz);
    }
    T *out = reinterpret_cast<T *>(a.dq) + row;
    for (int c = 0; c < 64; ++c) {
        if (c >= d)
            break;
        st(out + c, dq[c] * a.inv_sqrt_d);
    }
}

// One thread per (source, sample, channel), whole edge list.
template <typename T>
__global__ void __launch_bounds__(256) bwd_source_generic(const BwdArgs a)
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
    const T *DM = reinterpret_cast<const T *>(a.dm);
    float dk = 0.f, dv = 0.f;
    for (int j = a.csc_ptr[s]; j < a.csc_ptr[s + 1]; ++j) {
        const int t = a.csc_tgt[j];
        const int64_t o = ((int64_t)a.csc_pos[j] * a.B + b) * a.H + h;
        const int64_t r = ((int64_t)b * a.L + t) * a.E + c;
        const float2 v = get_pz<T>(a.PZ, o);
        dk = fmaf(v.y, ld(Q + r), dk);
        dv = fmaf(v.x, ld(DM + r), dv);
    }
    const int64_t w = ((int64_t)b * a.S + s) * a.E + c;
    st(reinterpret_cast<T *>(a.dk) + w, dk * a.inv_sqrt_d);
    st(reinterpret_cast<T *>(a.dv) + w, dv);
}

// ---- dx = sum_j dy_j W_j on the matrix cores ------------------------------
// Same scheme as the forward projections: the (transposed) weights sit in
// LDS in MFMA fragment order; each wavefront takes 16-row tiles (stride the
// grid), keeping the next tile's row fragments in flight, and stores whole
// 16-byte chunks of whole rows through a per-wavefront LDS staging area.

template <typename T> struct Frag;
template <> struct Frag<float> {      // v_mfma_f32_16x16x4f32, four per fragment
    static constexpr int kVec = 4, kStep = 16;
};
template <> struct Frag<uint16_t> {   // v_mfma_f32_16x16x32_bf16
    static constexpr int kVec = 8, kStep = 32;
};

template <typename T, int E, int NIN, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) bwd_rowmm(const RowMM a)
{
    constexpr int NKS = E / Frag<T>::kStep;
    constexpr int NT = E / 16;
    constexpr int PITCH = E * (int)sizeof(T) + 16;
    constexpr int CPR = E * (int)sizeof(T) / 16;
    constexpr int RPI = 64 / CPR;
    constexpr int KV = Frag<T>::kVec;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *wl = lds;
    char *stage = lds + NIN * NT * NKS * 1024 + (threadIdx.x >> 6) * (16 * PITCH);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // fragment (j, nt, ks), lane l: A[m][k] = W_j[k][m] for m = nt*16 + (l & 15),
    // k = ks * kStep + (l >> 4) * kVec + v
    // (per input map j its weight pointer is uniform; a thread's element loads
    // of up to two chunks are in flight together)
    constexpr int JCH = NT * NKS * 64;   // chunks per map
#pragma unroll
    for (int j = 0; j < NIN; ++j) {
        const T *W = reinterpret_cast<const T *>(a.w[j]);
        for (int c0 = threadIdx.x; c0 < JCH; c0 += 2 * WAVES * 64) {
            T v[2][KV];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = min(c0 + q * WAVES * 64, JCH - 1);
                const int f = c >> 6, l = c & 63;
                const int ks = f % NKS, nt = f / NKS;
                const int m = nt * 16 + (l & 15), k0 = ks * Frag<T>::kStep + (l >> 4) * KV;
#pragma unroll
                for (int i = 0; i < KV; ++i)
                    v[q][i] = W[(int64_t)(k0 + i) * E + m];
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = c0 + q * WAVES * 64;
                if (c < JCH)
                    *reinterpret_cast<uint4 *>(wl + (j * JCH + c) * 16) =
                        *reinterpret_cast<const uint4 *>(v[q]);
            }
        }
    }
    __syncthreads();

    const int64_t tile_rows = (int64_t)WAVES * 16;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    uint4 xf[NIN][NKS], xn[NIN][NKS];
    auto load_x = [&](int64_t tile, uint4 (&dst)[NIN][NKS]) {
        const int64_t r = tile * tile_rows + wid * 16 + lr;
        const int64_t rr = r < a.rows ? r : 0;
#pragma unroll
        for (int j = 0; j < NIN; ++j) {
            const T *xr = reinterpret_cast<const T *>(a.x[j]) + rr * E + lg * KV;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                dst[j][ks] = *reinterpret_cast<const uint4 *>(xr + ks * Frag<T>::kStep);
        }
    };
    const int cr = lane % CPR, rr = lane / CPR;
    // One tile from the x fragments in xf.
    auto process = [&](int64_t tile) {
        const int64_t row0 = tile * tile_rows + wid * 16;
#pragma unroll 2
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NIN; ++j) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const uint4 wf = *reinterpret_cast<const uint4 *>(
                        wl + (((j * NT + nt) * NKS + ks) * 64 + lane) * 16);
                    if constexpr (sizeof(T) == 2) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, xf[j][ks]),
                            acc, 0, 0, 0);
                    } else {
                        const float *wv = reinterpret_cast<const float *>(&wf);
                        const float *xv = reinterpret_cast<const float *>(&xf[j][ks]);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[q], xv[q], acc, 0, 0, 0);
                    }
                }
            }
            // lane holds output channels nt*16 + 4*lg + i of row lr
            if constexpr (sizeof(T) == 2) {
                char *d = stage + lr * PITCH + (nt * 16 + 4 * lg) * (int)sizeof(T);
                uint2 pk;
                pk.x = pack_bf16(acc[0], acc[1]);
                pk.y = pack_bf16(acc[2], acc[3]);
                *reinterpret_cast<uint2 *>(d) = pk;
            } else if (row0 + lr < a.rows) {
                // fp32: the lane's 16 contiguous bytes go straight out
                float4 *out = reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.y) +
                                                         (row0 + lr) * E + nt * 16 + 4 * lg);
                float4 v = make_float4(acc[0], acc[1], acc[2], acc[3]);
                if (a.accumulate) {
                    const float4 o = *out;
                    v = make_float4(v.x + o.x, v.y + o.y, v.z + o.z, v.w + o.w);
                }
                *out = v;
            }
        }
        if constexpr (sizeof(T) == 4)
            return;
        // a wavefront reads back only its own staged rows
        T *dst = reinterpret_cast<T *>(a.y) + cr * (16 / (int)sizeof(T));
#pragma unroll
        for (int it = 0; it < 16 / RPI; ++it) {
            const int lrow = it * RPI + rr;
            const int64_t r = row0 + lrow;
            if (r < a.rows) {
                uint4 v = *reinterpret_cast<const uint4 *>(stage + lrow * PITCH + cr * 16);
                uint4 *out = reinterpret_cast<uint4 *>(dst + r * E);
                if constexpr (sizeof(T) == 4) {
                    if (a.accumulate) {
                        const float4 o = *reinterpret_cast<const float4 *>(out);
                        v = make_uint4(__float_as_uint(__uint_as_float(v.x) + o.x),
                                       __float_as_uint(__uint_as_float(v.y) + o.y),
                                       __float_as_uint(__uint_as_float(v.z) + o.z),
                                       __float_as_uint(__uint_as_float(v.w) + o.w));
                    }
                }
                *out = v;
            }
        }
    };
    // Every tile but the last has a successor, whose fragments are loaded
    // before the tile is processed; the last one runs after the loop (a
    // conditional load in the loop makes the compiler wait for it at once).
    int64_t tile = blockIdx.x;
    if (tile < ntiles) {
        load_x(tile, xf);
        for (; tile + gridDim.x < ntiles; tile += gridDim.x) {
            load_x(tile + gridDim.x, xn);
            process(tile);
#pragma unroll
            for (int j = 0; j < NIN; ++j)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) xf[j][ks] = xn[j][ks];
        }
        process(tile);
    }
}

// Any embed_dim: one thread per (row, output channel).
template <typename T>
__global__ void __launch_bounds__(256) bwd_rowmm_generic(const RowMM a, int E)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t r = idx / E;
    const int i = (int)(idx - r * E);
    if (r >= a.rows)
        return;
    float acc = 0.f;
    for (int j = 0; j < a.nin; ++j) {
        const T *x = reinterpret_cast<const T *>(a.x[j]) + r * E;
        const T *w = reinterpret_cast<const T *>(a.w[j]) + i;
        for (int o = 0; o < E; ++o)
            acc = fmaf(ld(x + o), ld(w + (int64_t)o * E), acc);
    }
    T *y = reinterpret_cast<T *>(a.y) + r * E + i;
    if (a.accumulate)
        acc += ld(y);
    st(y, acc);
}

// ---- dW = G^T X and db = column sums of G ---------------------------------
// Workgroup = (row range, pair, 64 x 64 block of dW). Its four wavefronts
// take groups of 4 rows in turn; for v_mfma_f32_16x16x4f32 the lane (lr, lc)
// = (l >> 4, l & 15) supplies G[row lr][n0 + 4 lc + i] as the A value of
// tile i and X[row lr][k0 + 4 lc + i'] as the B value of tile i', so tile
// (i, i') accumulates dW[n0 + 4 m + i][k0 + 4 n + i'] at MFMA position
// (m, n): every load is a plain row-major read. The four wavefronts' sums
// meet in LDS and each workgroup writes one partial; a second kernel adds
// the partials in workgroup order.
constexpr int kWgPart = 64 * 64 + 64;   // floats per partial (dW block, db)

// Storage row of pair row r (the row list, where there is one).
__device__ inline int64_t wg_row(const WGradPair &p, int64_t r)
{
    if (!p.list)
        return r;
    const uint32_t rr = (uint32_t)r, n = (uint32_t)p.n;
    const uint32_t b = rr / n;
    return (int64_t)b * p.n_in + p.list[rr - b * n];
}

// Workgroup x of a weight-gradient launch: its pair, its rows, and the
// partial of 64 x 64 block z (partials of one pair and block are adjacent,
// in workgroup order).
struct WgSlice {
    WGradPair pr;
    int64_t r_beg, r_end;
    float *part0;   // partial of block 0; block z at + z * stride
    int64_t stride;
};
__device__ inline WgSlice wg_slice(const WGrad &a, int x)
{
    int i = 0;
    while (i + 1 < a.np && x >= a.off_p[i + 1])
        ++i;
    WgSlice w;
    w.pr = a.p[i];
    const int n = a.nwg_p[i], k = x - a.off_p[i];
    const int64_t per = (((w.pr.rows + n - 1) / n) + 15) & ~(int64_t)15;
    w.r_beg = (int64_t)k * per;
    w.r_end = w.r_beg + per < w.pr.rows ? w.r_beg + per : w.pr.rows;
    const int nz = (a.E / 64) * (a.E / 64);
    w.part0 = a.part + ((int64_t)a.off_p[i] * nz + k) * kWgPart;
    w.stride = (int64_t)n * kWgPart;
    return w;
}

template <typename T>
__global__ void __launch_bounds__(256) bwd_wgrad(const WGrad a)
{
    __shared__ float red[4][64 * 64];
    __shared__ float bred[4][64];
    const WgSlice ws = wg_slice(a, blockIdx.x);
    const WGradPair pr = ws.pr;
    const int zn = a.E / 64, zt = blockIdx.z;
    const int n0 = (zt / zn) * 64, k0 = (zt % zn) * 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lr = lane >> 4, lc = lane & 15;
    const int64_t r_beg = ws.r_beg, r_end = ws.r_end;
    const T *G = reinterpret_cast<const T *>(pr.g) + n0 + 4 * lc;
    const T *X = reinterpret_cast<const T *>(pr.x) + k0 + 4 * lc;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    auto load4 = [&](const T *p, float (&f)[4]) {
        if constexpr (sizeof(T) == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(p);
            f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
        } else {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            f[0] = __uint_as_float(v.x << 16);
            f[1] = __uint_as_float(v.x & 0xffff0000u);
            f[2] = __uint_as_float(v.y << 16);
            f[3] = __uint_as_float(v.y & 0xffff0000u);
        }
    };
    constexpr int UR = 4;   // row groups per wavefront per step
    for (int64_t r0 = r_beg + wid * 4; r0 < r_end; r0 += 16 * UR) {
        float g[UR][4], x[UR][4];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t r = r0 + 16 * u + lr;
            if (r < r_end) {
                const int64_t rr = wg_row(pr, r);
                load4(G + rr * a.E, g[u]);
                load4(X + rr * a.E, x[u]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) g[u][i] = x[u][i] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bs[i] += g[u][i];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(g[u][i], x[u][j], acc[i][j], 0, 0, 0);
            }
        }
    }
    // lane holds, for v < 4, MFMA position (m = 4 lr + v, n = lc)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wid][(4 * (4 * lr + v) + i) * 64 + 4 * lc + j] = acc[i][j][v];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bs[i] += __shfl_xor(bs[i], 16, 64);
        bs[i] += __shfl_xor(bs[i], 32, 64);
    }
    if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bred[wid][4 * lc + i] = bs[i];
    }
    __syncthreads();
    float *part = ws.part0 + zt * ws.stride;
    for (int e = threadIdx.x; e < 64 * 64; e += 256)
        part[e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
    if (threadIdx.x < 64) {
        const int e = threadIdx.x;
        part[64 * 64 + e] = ((bred[0][e] + bred[1][e]) + bred[2][e]) + bred[3][e];
    }
}

// fp32 with E = 128: the same MFMA scheme, but wavefront w takes block
// (w / 2, w % 2) of dW over all rows of the workgroup's range, so each row of
// G and X comes from HBM once per workgroup (the second wavefront's read of a
// half row is served by the CU's cache) and the partials need no reduction
// across wavefronts.
__global__ void __launch_bounds__(256) bwd_wgrad_quad(const WGrad a)
{
    const WgSlice ws = wg_slice(a, blockIdx.x);
    const WGradPair pr = ws.pr;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int lr = lane >> 4, lc = lane & 15;
    const int nb = wid >> 1, kb = wid & 1;
    const int64_t r_beg = ws.r_beg, r_end = ws.r_end;
    const float *G = reinterpret_cast<const float *>(pr.g) + 64 * nb + 4 * lc;
    const float *X = reinterpret_cast<const float *>(pr.x) + 64 * kb + 4 * lc;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    // Rows are loaded one step ahead (the loads of step k + 1 are in flight
    // during the matrix-core work of step k); a lane past the range loads
    // the range's last row and contributes zeros.
    constexpr int UR = 4;   // row groups of 4 per step
    float4 g[UR], x[UR], gn[UR], xn[UR];
    auto load = [&](int64_t r0, float4 (&gg)[UR], float4 (&xx)[UR]) {
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            int64_t r = r0 + 4 * u + lr;
            r = wg_row(pr, r < r_end ? r : r_end - 1);
            gg[u] = *reinterpret_cast<const float4 *>(G + r * a.E);
            xx[u] = *reinterpret_cast<const float4 *>(X + r * a.E);
        }
    };
    auto step = [&](int64_t r0) {
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const bool in = r0 + 4 * u + lr < r_end;
            const float gg[4] = {in ? g[u].x : 0.f, in ? g[u].y : 0.f, in ? g[u].z : 0.f,
                                 in ? g[u].w : 0.f};
            const float xx[4] = {in ? x[u].x : 0.f, in ? x[u].y : 0.f, in ? x[u].z : 0.f,
                                 in ? x[u].w : 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bs[i] += gg[i];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(gg[i], xx[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    if (r_beg < r_end) {
        load(r_beg, g, x);
        int64_t r0 = r_beg;
        for (; r0 + 4 * UR < r_end; r0 += 4 * UR) {
            load(r0 + 4 * UR, gn, xn);
            __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the work
            step(r0);
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                g[u] = gn[u];
                x[u] = xn[u];
            }
        }
        step(r0);
    }
    float *part = ws.part0 + (2 * nb + kb) * ws.stride;
    // lane holds, for v < 4, MFMA position (m = 4 lr + v, n = lc) of tile (i, j):
    // dW row 4 m + i, column 4 n + j
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<float4 *>(part + (4 * (4 * lr + v) + i) * 64 + 4 * lc) =
                make_float4(acc[i][0][v], acc[i][1][v], acc[i][2][v], acc[i][3][v]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bs[i] += __shfl_xor(bs[i], 16, 64);
        bs[i] += __shfl_xor(bs[i], 32, 64);
    }
    if (lr == 0)
        *reinterpret_cast<float4 *>(part + 64 * 64 + 4 * lc) = make_float4(bs[0], bs[1], bs[2], bs[3]);
}

// bf16: v_mfma_f32_16x16x32_bf16 contracts 8 consecutive rows per lane, so
// slabs of kWR rows of G and X are first written to LDS transposed (column-
// major, 2 RPT bytes per write); the workgroup covers a W x W block of dW
// (W = 64 ZN: ZN = 2 takes all of dW for E = 128, so every row of G and X is
// read once), wavefront w owns output rows 16 ZN w .. + 16 ZN - 1 and all W
// columns, so the partial needs no reduction across wavefronts. The next
// slab's loads are issued into the staging registers as soon as they have
// been written to LDS, and are in flight during the matrix-core work.
constexpr int kWR = 128;              // rows per slab
constexpr int kWP = kWR * 2 + 16;     // bytes per transposed column (padded)

__device__ inline uint32_t half16(const uint4 &u, int i)
{
    const uint32_t w = i < 2 ? u.x : i < 4 ? u.y : i < 6 ? u.z : u.w;
    return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int ZN>
__global__ void __launch_bounds__(256) bwd_wgrad_bf16(const WGrad a)
{
    constexpr int W = 64 * ZN;        // block width
    constexpr int CPR = W / 8;        // 16-byte chunks per slab row
    constexpr int RQ = 256 / CPR;     // threads per column chunk
    constexpr int RPT = kWR / RQ;     // slab rows per thread
    static_assert(RPT == 4 || RPT == 8, "slab rows per thread");
    static_assert(RQ * W * 4 <= W * kWP, "bias sums fit the G slab");
    __shared__ __attribute__((aligned(16))) char gt[W * kWP];
    __shared__ __attribute__((aligned(16))) char xt[W * kWP];
    const WgSlice ws = wg_slice(a, blockIdx.x);
    const WGradPair pr = ws.pr;
    const int zn = a.E / 64, zt = blockIdx.z;
    const int n0 = (zt / (zn / ZN)) * W, k0 = (zt % (zn / ZN)) * W;
    const int tid = threadIdx.x, rq = tid / CPR, cc = tid % CPR;
    const int lane = tid & 63, wid = tid >> 6;
    const int64_t r_beg = ws.r_beg, r_end = ws.r_end;
    const uint16_t *G = reinterpret_cast<const uint16_t *>(pr.g) + n0 + 8 * cc;
    const uint16_t *X = reinterpret_cast<const uint16_t *>(pr.x) + k0 + 8 * cc;
    f32x4 acc[ZN][4 * ZN];
#pragma unroll
    for (int mt = 0; mt < ZN; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4 * ZN; ++nt)
            acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        bsum[i] = 0.f;
    uint4 gv[RPT], xv[RPT];
    auto load = [&](int64_t r0) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int64_t r = r0 + RPT * rq + j;
            if (r < r_end) {
                const int64_t rr = wg_row(pr, r);
                gv[j] = ld16(G + rr * a.E);
                xv[j] = ld16(X + rr * a.E);
            } else {
                gv[j] = xv[j] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    if (r_beg < r_end)
        load(r_beg);
    for (int64_t r0 = r_beg; r0 < r_end; r0 += kWR) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                bsum[i] += __uint_as_float(half16(gv[j], i) << 16);
        __syncthreads();   // the previous slab's fragments are read
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int off = (8 * cc + i) * kWP + 2 * RPT * rq;
            if constexpr (RPT == 4) {
                *reinterpret_cast<uint2 *>(gt + off) =
                    make_uint2(half16(gv[0], i) | (half16(gv[1], i) << 16),
                               half16(gv[2], i) | (half16(gv[3], i) << 16));
                *reinterpret_cast<uint2 *>(xt + off) =
                    make_uint2(half16(xv[0], i) | (half16(xv[1], i) << 16),
                               half16(xv[2], i) | (half16(xv[3], i) << 16));
            } else {
                *reinterpret_cast<uint4 *>(gt + off) =
                    make_uint4(half16(gv[0], i) | (half16(gv[1], i) << 16),
                               half16(gv[2], i) | (half16(gv[3], i) << 16),
                               half16(gv[4], i) | (half16(gv[5], i) << 16),
                               half16(gv[6], i) | (half16(gv[7], i) << 16));
                *reinterpret_cast<uint4 *>(xt + off) =
                    make_uint4(half16(xv[0], i) | (half16(xv[1], i) << 16),
                               half16(xv[2], i) | (half16(xv[3], i) << 16),
                               half16(xv[4], i) | (half16(xv[5], i) << 16),
                               half16(xv[6], i) | (half16(xv[7], i) << 16));
            }
        }
        __syncthreads();
        if (r0 + kWR < r_end)
            load(r0 + kWR);
#pragma unroll
        for (int ks = 0; ks < kWR / 32; ++ks) {
            const int off = ks * 64 + 16 * (lane >> 4);
            uint4 af[ZN];
#pragma unroll
            for (int mt = 0; mt < ZN; ++mt)
                af[mt] = *reinterpret_cast<const uint4 *>(gt + (16 * (ZN * wid + mt) + (lane & 15)) * kWP + off);
#pragma unroll
            for (int nt = 0; nt < 4 * ZN; ++nt) {
                const uint4 bf = *reinterpret_cast<const uint4 *>(xt + (16 * nt + (lane & 15)) * kWP + off);
#pragma unroll
                for (int mt = 0; mt < ZN; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[mt]), __builtin_bit_cast(bf16x8, bf), acc[mt][nt], 0, 0, 0);
            }
        }
    }
    // partials stay in 64 x 64 blocks: block (n0 + 64 i, k0 + 64 j) of dW
    auto part_of = [&](int i, int j) {
        return ws.part0 + ((n0 / 64 + i) * zn + k0 / 64 + j) * ws.stride;
    };
    // lane holds position (m = 4 (lane >> 4) + v, n = lane & 15) of tile (ZN wid + mt, nt)
#pragma unroll
    for (int mt = 0; mt < ZN; ++mt) {
        const int row = 16 * (ZN * wid + mt) + 4 * (lane >> 4);
#pragma unroll
        for (int nt = 0; nt < 4 * ZN; ++nt) {
            float *part = part_of(row / 64, nt / 4);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                part[(row % 64 + v) * 64 + 16 * (nt % 4) + (lane & 15)] = acc[mt][nt][v];
        }
    }
    __syncthreads();   // the last slab's fragments are read
    float *bl = reinterpret_cast<float *>(gt);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        bl[rq * W + 8 * cc + i] = bsum[i];
    __syncthreads();
    if (tid < W) {
        float b = 0.f;
        for (int q = 0; q < RQ; ++q)
            b += bl[q * W + tid];
        // the same sums in every block column (only column 0 reaches db)
#pragma unroll
        for (int j = 0; j < ZN; ++j)
            part_of(tid / 64, j)[64 * 64 + tid % 64] = b;
    }
}

// Thread (e, q): partial element e summed over the workgroups w = q mod 4,
// then the four sums in order of q.
template <typename T>
__global__ void __launch_bounds__(256) bwd_wgrad_reduce(const WGrad a)
{
    __shared__ float red[4][64];
    const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + el;
    const WGradPair pr = a.p[blockIdx.z];
    const int zn = a.E / 64, zt = blockIdx.y;
    const int n0 = (zt / zn) * 64, k0 = (zt % zn) * 64;
    float acc = 0.f;
    if (e < kWgPart) {
        const int n = a.nwg_p[blockIdx.z];
        const float *part = a.part + ((int64_t)a.off_p[blockIdx.z] * gridDim.y + (int64_t)zt * n) * kWgPart + e;
#pragma unroll 8
        for (int w = q; w < n; w += 4)
            acc += part[(int64_t)w * kWgPart];
    }
    red[q][el] = acc;
    __syncthreads();
    if (q != 0 || e >= kWgPart)
        return;
    acc = ((red[0][el] + red[1][el]) + red[2][el]) + red[3][el];
    if (e < 64 * 64)
        st(reinterpret_cast<T *>(pr.dw) + (int64_t)(n0 + e / 64) * a.E + k0 + e % 64, acc);
    else if (k0 == 0 && pr.db)
        st(reinterpret_cast<T *>(pr.db) + n0 + (e - 64 * 64), acc);
}

// Any embed_dim: one workgroup per (output element, pair); element E*E + n
// is bias entry n.
template <typename T>
__global__ void __launch_bounds__(256) bwd_wgrad_generic(const WGrad a)
{
    __shared__ float red[256];
    const WGradPair pr = a.p[blockIdx.y];
    const int e = blockIdx.x, E = a.E;
    const bool bias = e >= E * E;
    if (bias && !pr.db)
        return;
    const int n = bias ? e - E * E : e / E, k = bias ? 0 : e % E;
    const T *G = reinterpret_cast<const T *>(pr.g);
    const T *X = reinterpret_cast<const T *>(pr.x);
    float acc = 0.f;
    for (int64_t r = threadIdx.x; r < pr.rows; r += 256) {
        const int64_t rr = wg_row(pr, r);
        acc = bias ? acc + ld(G + rr * E + n) : fmaf(ld(G + rr * E + n), ld(X + rr * E + k), acc);
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        st(reinterpret_cast<T *>(bias ? pr.db : pr.dw) + (bias ? n : (int64_t)n * E + k), red[0]);
}

inline unsigned grid(int64_t n) { return (unsigned)((n + 255) / 256); }

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

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
constexpr int kRowWaves = 8;

template <typename T, int E, int NIN>
constexpr size_t rowmm_lds()
{
    // bf16 rows are staged in LDS for whole-row 16-byte stores; fp32 lanes
    // store their 16 bytes directly
    return (size_t)NIN * (E / 16) * (E / Frag<T>::kStep) * 1024 +
           (sizeof(T) == 2 ? (size_t)kRowWaves * 16 * (E * sizeof(T) + 16) : 0);
}

template <typename T, int E, int NIN>
hipError_t run_rowmm(const RowMM &a, hipStream_t s)
{
    constexpr size_t lds = rowmm_lds<T, E, NIN>();
    static_assert(lds <= (size_t)kLdsBytes, "rowmm tile does not fit in LDS");
    const int64_t tile_rows = (int64_t)kRowWaves * 16;
    const int64_t ntiles = (a.rows + tile_rows - 1) / tile_rows;
    int per_cu = (int)(kLdsBytes / lds);
    per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
    int64_t g = (int64_t)cu_count() * per_cu;
    if (g > ntiles)
        g = ntiles;
    if (lds > 64 * 1024) {
        static bool raised = false;
        if (!raised) {
            hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(&bwd_rowmm<T, E, NIN, kRowWaves>),
                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
            if (e != hipSuccess)
                return e;
            raised = true;
        }
    }
    hipLaunchKernelGGL((bwd_rowmm<T, E, NIN, kRowWaves>), dim3((unsigned)g), dim3(kRowWaves * 64),
                       lds, s, a);
    return hipGetLastError();
}

// NIN inputs in one launch where the weights fit in LDS, else one launch
// per input accumulating into y (fp32 only).
template <typename T, int E>
hipError_t rowmm_e(const RowMM &a, hipStream_t s)
{
    constexpr bool fit2 = rowmm_lds<T, E, 2>() <= (size_t)kLdsBytes;
    constexpr bool fit3 = rowmm_lds<T, E, 3>() <= (size_t)kLdsBytes;
    if (a.nin == 1)
        return run_rowmm<T, E, 1>(a, s);
    if constexpr (fit3) {
        if (a.nin == 3)
            return run_rowmm<T, E, 3>(a, s);
    }
    if constexpr (fit2) {
        if (a.nin == 2)
            return run_rowmm<T, E, 2>(a, s);
    }
    for (int j = 0; j < a.nin; ++j) {
        RowMM one = a;
        one.nin = 1;
        one.x[0] = a.x[j];
        one.w[0] = a.w[j];
        one.accumulate = j > 0 ? 1 : a.accumulate;
        hipError_t e = run_rowmm<T, E, 1>(one, s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

bool bwd_edges_fast(int64_t E, int64_t H, pma_dtype dt, const void *q, const void *k,
                    const void *v, const void *mixed)
{
    const int64_t d = E / H, es = dt == PMA_BF16 ? 2 : 4, lph = d * es / 16;
    return (E * es) % 16 == 0 && (d * es) % 16 == 0 &&
           (lph == 1 || lph == 2 || lph == 4 || lph == 8 || lph == 16) && aligned16(q) &&
           aligned16(k) && aligned16(v) && aligned16(mixed);
}

pma_status launch_bwd_edges(const BwdArgs &a, pma_dtype dt, hipStream_t s)
{
    const int d = a.E / a.H;
    if (d > 64)
        return PMA_E_UNSUPPORTED;
    // (dm, dq, dk, dv come from the plan's 256-byte aligned scratch)
    const int lph = d * (dt == PMA_BF16 ? 2 : 4) / 16;
    const bool fast = bwd_edges_fast(a.E, a.H, dt, a.q, a.k, a.v, a.mixed) && aligned16(a.dm) &&
                      aligned16(a.dq) && aligned16(a.dk) && aligned16(a.dv);
    if (fast ? !a.mD : !a.PZ)
        return PMA_E_ARG;
    auto go = [&](auto tag) {
        using T = decltype(tag);
        if (!fast) {
            bwd_target_generic<T><<<grid((int64_t)a.L * a.B * a.H), 256, 0, s>>>(a);
            bwd_source_generic<T><<<grid((int64_t)a.S * a.B * a.E), 256, 0, s>>>(a);
            return;
        }
        const int cpr = a.E / Vec<T>::N;
        const int64_t nt = a.n_ttasks * a.B * cpr, ns = a.n_stasks * a.B * cpr;
        // a piece's lanes fill whole wavefronts: wavefront-uniform indices
        const bool uni = ((int64_t)a.B * cpr) % 64 == 0;
        // mask words by CSR position: whole wavefronts whose samples lie in
        // one 32-sample word (a power-of-two cpr >= 2: 64 / cpr samples
        // from a multiple of 64 / cpr; other cpr, e.g. 3 heads of one chunk,
        // make wavefronts straddle words, so those look bits up by source)
        const bool cm = uni && a.kpm_csr && cpr > 1 && (cpr & (cpr - 1)) == 0;
        // source pass with UNI: kBands interleaved runs of workgroups; within
        // a band the sample groups run one after another by default
        // (s_order 2; measured on MI355X: 100k-node source pass 2.47 ->
        // 2.28 ms, gene training step 0.94 -> 0.90 ms, bipartite level)
        int64_t per_band = 0;
        for (int k = 0; k < kBands; ++k) {
            const int64_t th = (a.s_band_off[k + 1] - a.s_band_off[k]) * a.B * cpr;
            per_band = std::max(per_band, (th + 255) / 256);
        }
        const unsigned gs_band = (unsigned)(per_band * kBands);
        // target pass order over sample groups (uni only)
        BwdArgs at = a;
        unsigned gt = grid(nt);
        const int G = (int)(((int64_t)a.B * cpr) / 64);
        at.t_groups = G;
        if (at.t_order < 0) {
            // Measured on MI355X, as for the forward's edge kernel: groups
            // pinned to XCDs pay at 8 groups (4% of a bipartite fp32 step;
            // at 4 groups they are level with the interleaved order); at 2
            // groups whose keys and values outgrow the 256 MB last-level
            // cache, groups in turn pay (1% of the 100k-node step).
            const uint64_t kv = (uint64_t)a.Skv * a.B * a.E * sizeof(T) * 2;
            at.t_order = G == 8 ? 1 : (G == 2 && kv > ((uint64_t)256 << 20) ? 2 : 0);
        }
        if (!uni || (at.t_order == 1 && 8 % G != 0))
            at.t_order = 0;
        if (at.t_pf < 0) {
            // Requesting a step's rows one step ahead doubles their registers
            // (4 wavefronts per SIMD instead of 7 for bf16). Measured on
            // MI355X: where the bf16 keys and values outgrow the 256 MB
            // last-level cache, more wavefronts with one step in flight each
            // win (100k-node target pass 1784 -> 1686 us); on the gene and
            // bipartite steps the two are level (within 1 %).
            const uint64_t kv = (uint64_t)a.Skv * a.B * a.E * sizeof(T) * 2;
            at.t_pf = sizeof(T) == 2 && kv > ((uint64_t)256 << 20) ? 0 : 1;
        }
        if (at.t_order != 0) {
            const int64_t gblocks = (a.n_ttasks * 64 + 255) / 256;   // per group
            at.t_gthreads = gblocks * 256;
            if (at.t_order == 1) {
                const int64_t per = 8 / G;   // XCDs per group
                gt = (unsigned)(8 * ((gblocks + per - 1) / per));
            } else {
                gt = (unsigned)(gblocks * G);
            }
        }
#define PMA_BWD_EDGE(L_)                                                            \
    case L_:                                                                       \
        if (uni) {                                                                 \
            if (cm && at.t_pf)                                                     \
                bwd_target_fast<T, L_, true, true><<<gt, 256, 0, s>>>(at);         \
            else if (cm)                                                           \
                bwd_target_fast<T, L_, true, true, false><<<gt, 256, 0, s>>>(at);  \
            else if (at.t_pf)                                                      \
                bwd_target_fast<T, L_, true><<<gt, 256, 0, s>>>(at);               \
            else                                                                   \
                bwd_target_fast<T, L_, true, false, false><<<gt, 256, 0, s>>>(at); \
            if (a.banded)                                                          \
                bwd_source_fast<T, L_, true><<<gs_band, 256, 0, s>>>(a);           \
            else                                                                   \
                bwd_source_fast<T, L_, true><<<grid(ns), 256, 0, s>>>(a);          \
        } else {                                                                   \
            bwd_target_fast<T, L_, false><<<grid(nt), 256, 0, s>>>(a);             \
            bwd_source_fast<T, L_, false><<<grid(ns), 256, 0, s>>>(a);             \
        }                                                                          \
        break;
        switch (lph) {
            PMA_BWD_EDGE(1)
            PMA_BWD_EDGE(2)
            PMA_BWD_EDGE(4)
            PMA_BWD_EDGE(8)
            PMA_BWD_EDGE(16)
        }
#undef PMA_BWD_EDGE
        // eight lanes per merged chunk where rows have many slots on average
        // (hub sources), one lane otherwise
        auto merge = [&](int64_t nsplit, int64_t nslots, int sources) {
            if (nsplit <= 0)
                return;
            if (nslots > 8 * nsplit)
                bwd_merge_fast<T, 8><<<grid(nsplit * a.B * cpr * 8), 256, 0, s>>>(a, sources);
            else
                bwd_merge_fast<T, 1><<<grid(nsplit * a.B * cpr), 256, 0, s>>>(a, sources);
        };
        merge(a.n_tsplit, a.n_tslots, 0);
        merge(a.n_ssplit, a.n_sslots, 1);
    };
    // The fast target pass and the merge share one ordering: the merge runs
    // after both edge passes, and reads only slots the target / source pass wrote.
    if (dt == PMA_BF16)
        go(uint16_t{});
    else
        go(float{});
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

size_t bwd_piece_scratch(const GraphDev &g, int64_t B, int64_t E)
{
    return ((size_t)g.n_slots * B * E + (size_t)g.n_sslots * B * 2 * E) * sizeof(float);
}

pma_status launch_rowmm(const RowMM &a, int64_t E, pma_dtype dt, hipStream_t s)
{
    if (a.rows <= 0)
        return PMA_OK;
    if (a.nin < 1 || a.nin > 3 || (a.accumulate && dt != PMA_F32))
        return PMA_E_ARG;
    bool al = aligned16(a.y);
    for (int j = 0; j < a.nin; ++j)
        al = al && aligned16(a.x[j]);
    hipError_t e;
    if (al && dt == PMA_BF16 && E == 64)
        e = rowmm_e<uint16_t, 64>(a, s);
    else if (al && dt == PMA_BF16 && E == 128)
        e = rowmm_e<uint16_t, 128>(a, s);
    else if (al && dt == PMA_F32 && E == 64)
        e = rowmm_e<float, 64>(a, s);
    else if (al && dt == PMA_F32 && E == 128)
        e = rowmm_e<float, 128>(a, s);
    else if (dt == PMA_BF16) {
        bwd_rowmm_generic<uint16_t><<<grid(a.rows * E), 256, 0, s>>>(a, (int)E);
        e = hipGetLastError();
    } else {
        bwd_rowmm_generic<float><<<grid(a.rows * E), 256, 0, s>>>(a, (int)E);
        e = hipGetLastError();
    }
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

namespace {
bool wgrad_fast(const WGrad &a, pma_dtype dt)
{
    if (a.E % 64 != 0)
        return false;
    const uintptr_t mask = 15;
    for (int i = 0; i < a.np; ++i)
        if (((uintptr_t)a.p[i].g | (uintptr_t)a.p[i].x) & mask)
            return false;
    return true;
}
}  // namespace

// Workgroups of a weight-gradient launch over all its pairs: one per 256
// rows, at most 2048 / (number of 64 x 64 blocks of dW), i.e. at most 2048
// partial blocks; launch_wgrad deals them to the pairs in proportion to their
// rows, at least one each (so at most np more).
static int64_t wgrad_budget(int64_t E, int64_t rows)
{
    const int64_t nz = (E / 64) * (E / 64);
    int64_t cap = 2048 / (nz > 0 ? nz : 1);
    if (cap < 1)
        cap = 1;
    int64_t n = (rows + 255) / 256;
    if (n < 1)
        n = 1;
    return n < cap ? n : cap;
}

size_t wgrad_scratch(int64_t E, int np, int64_t max_rows)
{
    if (E % 64 != 0)
        return 0;
    const int64_t nz = (E / 64) * (E / 64);
    return (size_t)(wgrad_budget(E, np * max_rows) + np) * nz * kWgPart * sizeof(float);
}

pma_status launch_wgrad(WGrad a, pma_dtype dt, hipStream_t s)
{
    if (a.np <= 0)
        return PMA_OK;
    int64_t rows = 0;
    for (int i = 0; i < a.np; ++i)
        rows += a.p[i].rows;
    const bool bf = dt == PMA_BF16;
    if (wgrad_fast(a, dt)) {
        const int64_t budget = wgrad_budget(a.E, rows);
        a.nwg = 0;
        for (int i = 0; i < a.np; ++i) {
            const int64_t n = rows > 0 ? budget * a.p[i].rows / rows : 0;
            a.nwg_p[i] = (int)(n > 1 ? n : 1);
            a.off_p[i] = a.nwg;
            a.nwg += a.nwg_p[i];
        }
        const int zn = a.E / 64;
        const dim3 g1((unsigned)a.nwg, 1, (unsigned)(zn * zn));
        const dim3 g2((unsigned)((kWgPart + 63) / 64), (unsigned)(zn * zn), (unsigned)a.np);
        if (bf) {
            if (zn == 2)   // one workgroup reads its rows once for all of dW
                bwd_wgrad_bf16<2><<<dim3(g1.x, g1.y, 1), 256, 0, s>>>(a);
            else
                bwd_wgrad_bf16<1><<<g1, 256, 0, s>>>(a);
            bwd_wgrad_reduce<uint16_t><<<g2, 256, 0, s>>>(a);
        } else {
            if (zn == 2)
                bwd_wgrad_quad<<<dim3(g1.x, g1.y, 1), 256, 0, s>>>(a);
            else
                bwd_wgrad<float><<<g1, 256, 0, s>>>(a);
            bwd_wgrad_reduce<float><<<g2, 256, 0, s>>>(a);
        }
    } else {
        const dim3 g((unsigned)(a.E * a.E + a.E), (unsigned)a.np);
        if (bf)
            bwd_wgrad_generic<uint16_t><<<g, 256, 0, s>>>(a);
        else
            bwd_wgrad_generic<float><<<g, 256, 0, s>>>(a);
    }
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
