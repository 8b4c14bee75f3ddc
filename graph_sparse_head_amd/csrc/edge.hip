// Score, softmax and mix over the live edges (kpnn2 PackedMultiheadAttention
// page, "Notes" steps 2-4): for target t, head h and sample b,
//   score[e] = dot(q_h[t], k_h[s_e]) / sqrt(d) for the edges e into t,
//   weight[e] = softmax of those scores over the edges into t only,
//   mixed_h[t] = sum_e weight[e] v_h[s_e],
// and a target without edges mixes to zeros (same page, paragraph after the
// steps). The page states the result; how it is evaluated here is this
// library's design:
//   * no per-edge score array: a running maximum and running sum (online
//     softmax) rescale the partial mix as edges stream past, evaluated in base
//     2 (scores pre-multiplied by log2(e) / sqrt(d), weights from exp2);
//   * one wavefront handles one piece of a target's edge list for a group of
//     samples; each lane owns a 16-byte chunk of one sample's row, so a head
//     spans LPH = d / CH adjacent lanes and its dot product is reduced with
//     DPP lane swaps;
//   * targets longer than the plan's chunk are split into pieces whose
//     (max, sum, partial mix) are merged afterwards in a fixed order;
//   * with need_weights the log2-domain scores are stored per CSR position
//     and normalised once the final (max, sum) of each target is known;
//   * at embed_dim 64 (inference) the same kernel applies out_proj to the
//     mixed rows it has just made and, for bf16, also projects each target's
//     q from its query tokens at the start of the piece (step 1), with Wq and
//     Wo held in LDS as matrix-core fragments: neither q nor the mixed rows
//     travel through memory.
//
// Workspace layouts: q, keys/values and mixed rows are addressed through
// element strides (Layout); part_acc[slot][B][E], part_ml[slot][B][H][2],
// stat_ml[L][B][H][2], scores[nnz][B][H].
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "pma_internal.h"

namespace pma {
namespace {

struct EdgeK {
    const int32_t *csr_src, *csr_tgt, *csr_eid;
    const int32_t *task_target, *task_begin, *task_end, *task_slot;
    const int32_t *split_target, *split_slot0, *split_count;
    int64_t n_tasks, n_split, n_slots;
    int B, E, H, d;
    int64_t nnz;
    int passes;          // wavefronts per piece (sample groups)
    // n / passes and n / (E / CH) as (n * m) >> sh for n < 2^31 (see magic31)
    uint32_t pass_m, cpr_m;
    int pass_sh, cpr_sh;
    // 1: sample group fixed per XCD (passes divides 8); 2: sample groups in
    // turn (wavefront w serves group w / tstride), 0: interleaved
    int xcd_map;
    uint32_t xcd_per;    // 8 / passes
    uint32_t tstride;    // pieces between a wavefront's consecutive pieces
    uint32_t ts_m;       // n / tstride as (n * ts_m) >> ts_sh
    int ts_sh;
    // key_padding_mask as bits: source s, sample b at bit b % 64 of
    // kpm_bits[s * kpm_words + b / 64] (source id from orig_src); a set bit
    // leaves the key out. nullptr: no mask.
    const uint64_t *kpm_bits;
    int kpm_words;
    const int32_t *orig_src;
    // the same bits by CSR position in 32-bit words: bit b % 32 of
    // kpm_csr[p * kpm_w32 + b / 32] for the edge at p (edge_fast reads one
    // uniform word per edge, two when a wavefront spans 64 samples)
    const uint32_t *kpm_csr;
    int kpm_w32;
    int nt;              // bit 0: non-temporal q loads, bit 1: non-temporal mixed / out stores
    float scale;         // log2(e) / sqrt(d)
    Layout lay;
    const void *qt, *kv;
    uint64_t kv_bytes;   // size of the key/value workspace
    void *mixed;
    float *part_acc, *part_ml, *stat_ml, *scores, *weights;
    int average;
    // out_proj in the epilogue (fuse_out): caller's Wo, bo, out (B, L, E)
    int fuse_out, L;
    const void *wo, *bo;
    void *out;
    // q projection in the prologue (fuse_in): qt / lay address the caller's
    // query tokens and each piece projects its target's rows with Wq, bq
    int fuse_in;
    const void *wq, *bq;
    // hot-row cache (edge_fast with HOT slots): hot_src[i] is the key/value
    // row cached in slot i; hot_csr is csr_src with ~slot in place of the
    // cached rows (passed as the gather index of that kernel only)
    const int32_t *hot_src, *hot_csr;
    int n_hot;
    // split targets merged by the edge kernel itself (see edge_fast):
    // allow_coop where every split target has at most 4 pieces; coop_blocks
    // leading workgroups of the launch serve them (0: merge launch instead)
    const int32_t *row_ptr;
    int allow_coop;
    uint32_t coop_blocks;
};

__device__ inline float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ inline uint4 load_nt(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store_nt(void *p, const uint4 &u)
{
    __builtin_nontemporal_store(u32x4_t{u.x, u.y, u.z, u.w}, reinterpret_cast<u32x4_t *>(p));
}

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ inline uint16_t f2bf(float f) { return (uint16_t)(pack_bf16(f, 0.f) & 0xffffu); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// floor(n / d) for n < 2^31 from a host-made multiplier (magic31)
__device__ inline uint32_t div31(uint32_t n, uint32_t m, int sh)
{
    return (uint32_t)(((uint64_t)n * m) >> sh);
}

template <int CTRL> __device__ inline float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of G lanes; every lane of the group gets the
// same bits (each step adds a lane to its partner, and fp addition commutes).
template <int G> __device__ inline float group_sum(float x)
{
    if constexpr (G >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (G >= 16) x += dpp<0x140>(x); // row_mirror
    if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// CH elements of type T in one 16-byte word, widened to fp32 on use.
template <typename T, int CH> struct Chunk {
    uint4 u;
    __device__ inline void load(const T *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ inline void zero() { u = make_uint4(0, 0, 0, 0); }
    __device__ inline uint32_t word(int k) const
    {
        return k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
    }
    __device__ inline float operator[](int i) const
    {
        if constexpr (sizeof(T) == 4) {
            static_assert(CH == 4, "fp32 chunks are 16 bytes");
            return __uint_as_float(word(i));
        } else {
            static_assert(CH == 8, "bf16 chunks are 16 bytes");
            const uint32_t w = word(i >> 1);
            return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        }
    }
};

template <typename T, int CH> __device__ inline void store_chunk(T *p, const float *v, bool nt = false)
{
    uint4 u;
    if constexpr (sizeof(T) == 4) {
        u = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                       __float_as_uint(v[3]));
    } else {
        u.x = pack_bf16(v[0], v[1]);
        u.y = pack_bf16(v[2], v[3]);
        u.z = pack_bf16(v[4], v[5]);
        u.w = pack_bf16(v[6], v[7]);
    }
    if (nt)
        store_nt(p, u);
    else
        *reinterpret_cast<uint4 *>(p) = u;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// out = mixed Wo^T + bo (kpnn2 page, "Notes" step 5) for the samples of one
// wavefront, straight from edge_fast's lane layout (lane = sample * CPR +
// chunk, chunk = CH channels of mixed). MFMA 16x16 tiles: the A operand is
// Wo, the B operand mixed^T with one column per sample. At k-step ks, lane
// group g feeds chunk 4 ks + g of sample l % 16, fetched from its owner lane
// with ds_bpermute; Wo is read in the same (natural) channel order. Row r of
// n-tile nt is output channel (E/4)(r/4) + 4 nt + r%4, so each lane ends with
// E/4 contiguous output channels of one sample and stores whole 16-byte words.
// Wo as MFMA A fragments in LDS: fragment (n-tile nt, k-group kg) is 64
// lanes x 16 bytes at byte ((nt * KG + kg) * 64 + lane) * 16, lane l holding
// output channel (E/4)(l%16 / 4) + 4 nt + l%4 at channels (4 kg + l/16) * CH.
// (Workgroups of 256 threads: each thread's loads are issued together, then
// stored, so staging costs one memory round trip.)
template <typename T, int CH, int E>
__device__ inline void stage_w(const void *w, const void *b, char *wlds)
{
    constexpr int KG = E / (4 * CH), NT = E / 16, CPL = E / 4;
    constexpr int NF = NT * KG * 64 / 256;   // fragment chunks per thread
    static_assert(NT * KG * 64 % 256 == 0 && E <= 256, "256 threads stage whole fragments");
    const T *W = reinterpret_cast<const T *>(w);
    uint4 v[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = threadIdx.x + 256 * i;
        const int lane = f & 63, fk = f >> 6, kg = fk % KG, nt = fk / KG;
        const int n = lane & 15, g = lane >> 4;
        const int orow = CPL * (n >> 2) + 4 * nt + (n & 3);
        v[i] = *reinterpret_cast<const uint4 *>(W + orow * E + (4 * kg + g) * CH);
    }
    // bias as fp32 after the fragments (zeros without bias)
    const T *bias = reinterpret_cast<const T *>(b);
    const int c = threadIdx.x;
    float bv = 0.f;
    if (bias && c < E) {
        if constexpr (sizeof(T) == 2)
            bv = bf2f(bias[c]);
        else
            bv = bias[c];
    }
#pragma unroll
    for (int i = 0; i < NF; ++i)
        *reinterpret_cast<uint4 *>(wlds + (threadIdx.x + 256 * i) * 16) = v[i];
    if (c < E)
        reinterpret_cast<float *>(wlds + NT * KG * 64 * 16)[c] = bv;
}

// bytes of one staged E x E matrix with its bias
template <typename T, int E> constexpr int staged_bytes() { return E * E * (int)sizeof(T) + 4 * E; }

template <typename T, int CH, int E>
__device__ inline void stage_wo(const EdgeK &a, char *wlds)
{
    stage_w<T, CH, E>(a.wo, a.bo, wlds);
}

// y = x W^T + bias for the samples of one wavefront with W staged by
// stage_w; w holds this lane's 16-byte chunk of x (lane = sample * CPR +
// chunk). Lane (n, g) = (lane % 16, lane / 16) gets output channels
// CPL g .. CPL g + CPL - 1 of sample n as T words in ow (zeros-in rows for
// n >= samples per wavefront).
template <typename T, int CH, int E, bool OPAQUE = false>
__device__ inline void proj_wave(const uint32_t *w, int lane, const char *wlds,
                                 uint32_t *ow)
{
    // This lane's byte offsets of its fragments and of its bias slice. With
    // OPAQUE they are hidden from the optimiser, so that a call inside a loop
    // re-reads the LDS each time instead of keeping the whole matrix in
    // registers across the loop.
    constexpr int CPR = E / CH;     // chunks per sample row
    constexpr int SPW = 64 / CPR;   // samples per wavefront
    constexpr int NT = E / 16;
    constexpr int CPL = E / 4;      // output channels per lane
    uint32_t fo = (uint32_t)lane * 16, bo = (uint32_t)(lane >> 4) * CPL * 4;
    if constexpr (OPAQUE) {
        asm volatile("" : "+v"(fo));
        asm volatile("" : "+v"(bo));
    }
    const int n = lane & 15, g = lane >> 4;
    const bool has = n < SPW;
    // k-groups: 32 channels (bf16) or 16 channels (fp32) per group
    constexpr int KG = E / (4 * CH);
    uint32_t bw[KG][4];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
        const int src = has ? n * CPR + 4 * kg + g : lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = __builtin_amdgcn_ds_bpermute(src << 2, (int)w[j]);
            bw[kg][j] = has ? (uint32_t)v : 0u;
        }
    }
    const float *bl = reinterpret_cast<const float *>(wlds + NT * KG * 64 * 16);
    // one n-tile at a time; results packed into T words as they are made
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float4 b4 = *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(bl) + bo + 16 * nt);
        f32x4_t acc = {b4.x, b4.y, b4.z, b4.w};   // bias first
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const uint4 wa = *reinterpret_cast<const uint4 *>(wlds + fo + (nt * KG + kg) * 1024);
            if constexpr (sizeof(T) == 2) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, wa),
                    __builtin_bit_cast(bf16x8_t, make_uint4(bw[kg][0], bw[kg][1], bw[kg][2], bw[kg][3])),
                    acc, 0, 0, 0);
            } else {
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wa.x), __uint_as_float(bw[kg][0]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wa.y), __uint_as_float(bw[kg][1]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wa.z), __uint_as_float(bw[kg][2]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(wa.w), __uint_as_float(bw[kg][3]), acc, 0, 0, 0);
            }
        }
        float o[4] = {acc[0], acc[1], acc[2], acc[3]};
        if constexpr (sizeof(T) == 2) {
            ow[2 * nt] = pack_bf16(o[0], o[1]);
            ow[2 * nt + 1] = pack_bf16(o[2], o[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ow[4 * nt + i] = __float_as_uint(o[i]);
        }
    }
}

template <typename T, int CH, int E, bool W32>
__device__ inline void out_proj_wave(const EdgeK &a, const float *mix, int lane, int t,
                                     int b_first, const char *wlds)
{
    constexpr int SPW = 64 / (E / CH);
    constexpr int CPL = E / 4;
    constexpr int OW = CPL * (int)sizeof(T) / 4;   // 32-bit words of this lane's output
    uint32_t w[4];                  // this lane's mixed chunk as 16 bytes of T
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16(mix[2 * j], mix[2 * j + 1]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = __float_as_uint(mix[j]);
    }
    uint32_t ow[OW];
    proj_wave<T, CH, E>(w, lane, wlds, ow);
    const int n = lane & 15, g = lane >> 4;
    const int b = b_first + n;
    if (n >= SPW || b >= a.B)
        return;
    T *o = reinterpret_cast<T *>(a.out);
    if (W32)   // out under 2 GiB: 32-bit element offset
        o += ((uint32_t)b * (uint32_t)a.L + (uint32_t)t) * (uint32_t)E + CPL * g;
    else
        o += ((int64_t)b * a.L + t) * E + CPL * g;
    char *dst = reinterpret_cast<char *>(o);
#pragma unroll
    for (int k = 0; k < OW / 4; ++k) {
        const uint4 v = make_uint4(ow[4 * k], ow[4 * k + 1], ow[4 * k + 2], ow[4 * k + 3]);
        if (a.nt & 2)
            store_nt(dst + 16 * k, v);
        else
            *reinterpret_cast<uint4 *>(dst + 16 * k) = v;
    }
}

// q = x Wq^T + bq (kpnn2 page, "Notes" step 1) for the current target of
// one wavefront, from the lane's chunk of its own x row; returns the lane's
// chunk of q in the lane layout (lane = sample * CPR + chunk), rounded to T
// as a separate projection would store it. proj_wave leaves channels
// CPL g .. of sample n on lane 16 g + n; each lane fetches its CH channels
// from there (every word, then the ones at its offset are kept).
template <typename T, int CH, int E>
__device__ inline uint4 q_proj_wave(const uint4 &x, int lane, const char *wlds)
{
    constexpr int CPR = E / CH, CPL = E / 4;
    constexpr int OW = CPL * (int)sizeof(T) / 4;
    constexpr int PARTS = CPL / CH;   // CH-channel chunks per MFMA lane
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t ow[OW];
    proj_wave<T, CH, E, true>(w, lane, wlds, ow);
    const int s = lane / CPR, c = lane % CPR;
    const int src = (c / PARTS) * 16 + s, part = c % PARTS;
    uint32_t r[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < PARTS; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)ow[4 * k + j]);
            r[j] = part == k ? v : r[j];
        }
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Merge of split target k's pieces for sample group `pass` (kpnn2 page,
// "Notes" step 3 over the union of the pieces' edges): each piece left its
// (max, sum) per head and its unnormalised mix in its partial slot; they are
// combined in slot order against the largest maximum. `staged` is called by
// every thread once the first PF pieces' partials are requested (merge_fast
// stages Wo there, so that their memory latency overlaps the staging and its
// barrier; in the edge kernel Wo is staged already, and holding partials
// there would raise the register count of the whole kernel). Lanes of an
// invalid unit return after it.
template <typename T, int CH, int LPH, int E_FUSE, int PF, typename F>
__device__ inline void merge_split(const EdgeK &a, uint32_t k, int pass, bool valid, int lane,
                                   const char *wlds, F &&staged)
{
    const int B = a.B, E = a.E, H = a.H;
    const int cpr = E / CH;
    const int c = pass * 64 + lane;
    const bool active = valid && c < B * cpr;
    const int b = active ? (int)div31(c, a.cpr_m, a.cpr_sh) : 0, cr = c - b * cpr,
              col = active ? cr * CH : 0;
    const int h = active ? cr / LPH : 0;
    const int t = valid ? a.split_target[k] : 0, s0 = valid ? a.split_slot0[k] : 0;
    const int n = active ? a.split_count[k] : 0;
    auto ml_at = [&](int j) {
        return *reinterpret_cast<const float2 *>(a.part_ml + (((int64_t)(s0 + j) * B + b) * H + h) * 2);
    };
    auto acc_at = [&](int j) {
        return reinterpret_cast<const float4 *>(a.part_acc + ((int64_t)(s0 + j) * B + b) * E + col);
    };
    float2 pml[PF];
    float4 pacc[PF][CH / 4];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        if (j < n) {
            pml[j] = ml_at(j);
#pragma unroll
            for (int q = 0; q < CH / 4; ++q) pacc[j][q] = acc_at(j)[q];
        }
    }
    staged();
    if (!valid)
        return;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < PF; ++j)
        if (j < n) M = fmaxf(M, pml[j].x);
    for (int j = PF; j < n; ++j)
        M = fmaxf(M, ml_at(j).x);
    float l = 0.f, acc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[i] = 0.f;
    // (a piece whose keys are all masked has l = 0 and m = -inf)
    auto add = [&](const float2 ml, const float4 *v) {
        const float w = ml.y > 0.f ? fast_exp2(ml.x - M) : 0.f;
        l = fmaf(ml.y, w, l);
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) {
            acc[4 * q + 0] = fmaf(v[q].x, w, acc[4 * q + 0]);
            acc[4 * q + 1] = fmaf(v[q].y, w, acc[4 * q + 1]);
            acc[4 * q + 2] = fmaf(v[q].z, w, acc[4 * q + 2]);
            acc[4 * q + 3] = fmaf(v[q].w, w, acc[4 * q + 3]);
        }
    };
#pragma unroll
    for (int j = 0; j < PF; ++j)
        if (j < n) add(pml[j], pacc[j]);
    for (int j = PF; j < n; ++j) {
        float4 v[CH / 4];
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) v[q] = acc_at(j)[q];
        add(ml_at(j), v);
    }
    const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
    float out[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) out[i] = acc[i] * inv;
    if (active && a.stat_ml && (lane % LPH) == 0) {
        float *st = a.stat_ml + (((int64_t)t * B + b) * H + h) * 2;
        st[0] = M;
        st[1] = l;
    }
    if constexpr (E_FUSE > 0) {
        if (a.fuse_out) {
            out_proj_wave<T, CH, E_FUSE, false>(a, out, lane, t, pass * (64 / (E_FUSE / CH)), wlds);
            return;
        }
    }
    if (active)
        store_chunk<T, CH>(reinterpret_cast<T *>(a.mixed) + t * a.lay.m_t + b * a.lay.m_b + col, out);
}

// Hot-row cache slot: the 16-byte key chunks of a wavefront's 64 lanes, then
// their value chunks, for one source row.
constexpr uint32_t kHotSlot = 2048;

// Fast path: d = CH * LPH with 16-byte chunks.
//
// Per edge the source's key/value row offset is wave-uniform: one scalar
// multiply gives it, and each lane adds its fixed offset inside the row. When
// every tensor the kernel addresses is under 2 GiB the gathers are buffer loads whose
// scalar offset is that product (no vector address arithmetic; a read past
// the buffer returns zeros instead of faulting); otherwise they are global
// loads from a uniform 64-bit base. Lanes past the last chunk read lane 0's
// address and discard the data. bf16 scores use v_dot2 on the stored bf16 q
// and k words (fp32 products and sums) and are scaled afterwards. Edges run U
// at a time, the remainder one at a time.
// KPM: 0 no mask, 1 one mask word per position covers the wavefront's
// samples, 2 two words (a wavefront's samples may straddle a multiple of
// 32: 64 samples per wavefront, or a row of chunks that is not a power of
// two, so that wavefronts start mid-row); each lane picks the word of its
// own sample.
template <typename T, int CH, int LPH, bool W32, bool SC, int KPM, bool HT = false,
          bool HS = false>
struct EdgeLane {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
    static constexpr bool BF = sizeof(T) == 2;

    const EdgeK &a;
    const int32_t *src;   // gather rows, from a noalias kernel argument
    const uint32_t *kbits;  // mask bits by CSR position, from a noalias kernel argument
    uint32_t kword;         // first 32-bit word of this wavefront's samples at a position
    bool khi;               // this lane's sample is in the word after kword (KPM == 2)
    int B, b, h;
    bool active, head_lead;
    Chunk<T, CH> q;
    float qf[BF ? 1 : CH];
    float l = 0.f, acc[CH];
    const char *kvb;
    __amdgpu_buffer_rsrc_t rsrc;
    typedef typename std::conditional<W32, uint32_t, uint64_t>::type Off;
    uint64_t row2;
    Off loff, vloff;   // this lane's key and value chunk inside a source's rows
    uint32_t sc_lane, sc_edge;            // scores element offsets: this lane's, per edge
    const char *hl;                       // this lane's key chunk in hot-row slot 0 (LDS)

    __device__ EdgeLane(const EdgeK &a_) : a(a_) {}

    // a cached row (index ~slot): key and value chunks from LDS
    __device__ inline void gather_hot(int s, Chunk<T, CH> &k, Chunk<T, CH> &v) const
    {
        const char *h = hl + (uint32_t)(~s) * kHotSlot;
        k.u = *reinterpret_cast<const uint4 *>(h);
        v.u = *reinterpret_cast<const uint4 *>(h + 1024);
    }

    __device__ inline void gather(int s, Chunk<T, CH> &k, Chunk<T, CH> &v) const
    {
        if constexpr (HT) {
            if (s < 0) {   // wave-uniform
                gather_hot(s, k, v);
                return;
            }
        }
        gather_cold(s, k, v);
    }

    __device__ inline void gather_cold(int s, Chunk<T, CH> &k, Chunk<T, CH> &v) const
    {
        if constexpr (W32) {
            const uint32_t so = (uint32_t)s * (uint32_t)row2;   // uniform
            const u32x4 kw = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)loff, so, 0);
            const u32x4 vw = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)vloff, so, 0);
            k.u = make_uint4(kw.x, kw.y, kw.z, kw.w);
            v.u = make_uint4(vw.x, vw.y, vw.z, vw.w);
        } else {
            const char *base = kvb + (uint64_t)s * row2;        // uniform
            k.u = *reinterpret_cast<const uint4 *>(base + loff);
            v.u = *reinterpret_cast<const uint4 *>(base + vloff);
        }
    }

    // N edges starting at CSR position p, all of them live
    // First bf16 product of a score with a zero accumulator (the VOP3 form
    // takes the 0 as an inline constant; v_dot2c would need it in a register).
    __device__ static inline float dot2_first(uint32_t x, uint32_t y)
    {
        float r;
        asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(y));
        return r;
    }

    // N live edges starting at CSR position p.
    //
    // Softmax reference: the weight of an edge is exp2(score - ms), scores in
    // log2 units. The reference ms moves up to the running maximum only when
    // some lane's maximum exceeds it by more than kLazy, so most steps skip
    // the rescale of the partial sums; weights stay below 2^kLazy. Any
    // reference gives the same normalised result (the sum and the mix are
    // both relative to it), and a lone edge still gets weight exp2(0) = 1.
    static constexpr float kLazy = 8.f;
    float smul, ms = -INFINITY;
    bool fresh = true;

    // N live edges starting at CSR position p; with PRE the source ids of the
    // next N edges are read into nsrc after this step's gathers are issued
    // (so that the next step's gathers need not wait for them).
    int nsrc[4];

    // Scores held for storing (SC with HS): hn of them from CSR position hp.
    // The kernel asks for it where the four registers are free; elsewhere
    // holding them spills (4-36 registers) and each step's scores are stored
    // at once.
    static constexpr bool HOLD = SC && HS;
    float hsc[HOLD ? 4 : 1];
    int hp = 0, hn = 0;
    __device__ inline void flush_scores()
    {
        if constexpr (HOLD) {
            if (active && head_lead) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (u < hn) {
                        // (a store through a buffer resource would hide from
                        // alias analysis that csr_src is never written, and
                        // turn its uniform scalar loads into vector loads)
                        if constexpr (W32)
                            a.scores[(uint32_t)(hp + u) * sc_edge + sc_lane] = hsc[u];
                        else
                            a.scores[(((int64_t)(hp + u)) * B + b) * a.H + h] = hsc[u];
                    }
                }
            }
            hn = 0;
        }
    }

    template <int N, bool PRE = false> __device__ inline void step(int p, const int *csrc = nullptr)
    {
        // mask words first, as uniform (scalar) loads in flight with the
        // gathers; with 64 samples per wavefront both words of a position
        uint32_t mlo[N], mhi[N];
        if constexpr (KPM > 0) {
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const uint32_t i = __builtin_amdgcn_readfirstlane(
                    (uint32_t)(p + u) * (uint32_t)a.kpm_w32 + kword);
                mlo[u] = kbits[i];
                if constexpr (KPM == 2)
                    mhi[u] = kbits[i + 1];
            }
        }
        Chunk<T, CH> kk[N], vv[N];
        if constexpr (HT) {
            // A row lists its cached sources first: a step is all cached, all
            // from memory, or (once per piece) the boundary between them.
            int sv[N];
#pragma unroll
            for (int u = 0; u < N; ++u) sv[u] = src[p + u];
            if (sv[N - 1] < 0) {
#pragma unroll
                for (int u = 0; u < N; ++u) gather_hot(sv[u], kk[u], vv[u]);
            } else if (sv[0] >= 0) {
#pragma unroll
                for (int u = 0; u < N; ++u) gather_cold(sv[u], kk[u], vv[u]);
            } else {
#pragma unroll
                for (int u = 0; u < N; ++u) gather(sv[u], kk[u], vv[u]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u) gather(csrc ? csrc[u] : src[p + u], kk[u], vv[u]);
        }
        if constexpr (PRE) {
#pragma unroll
            for (int u = 0; u < N; ++u) nsrc[u] = src[p + N + u];
        }
        float sc[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            float dot;
            if constexpr (BF) {
                dot = dot2_first(q.word(0), kk[u].word(0));
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.word(k)),
                                                          __builtin_bit_cast(bf16x2, kk[u].word(k)),
                                                          dot, false);
            } else {
                dot = 0.f;
#pragma unroll
                for (int i = 0; i < CH; ++i) dot = fmaf(qf[i], kk[u][i], dot);
            }
            dot = group_sum<LPH>(dot);
            if constexpr (BF) dot *= smul;   // fp32 q carries the scale already
            sc[u] = dot;
        }
        if constexpr (KPM > 0) {   // masked keys leave the softmax
            // one or two uniform 32-bit words per edge hold the bits of all
            // the wavefront's samples
#pragma unroll
            for (int u = 0; u < N; ++u) {
                uint32_t w = mlo[u];
                if constexpr (KPM == 2)
                    w = khi ? mhi[u] : w;
                if ((w >> (b & 31)) & 1u)
                    sc[u] = -INFINITY;
            }
        }
        if constexpr (HOLD) {
            // The previous step's scores go out now that this step's gathers
            // are issued (vector memory operations complete in order: stored
            // before them, they would hold back their use; bipartite edge
            // kernel 347 -> 341 us); this step's are held until the next step
            // or the end of the piece.
            flush_scores();
#pragma unroll
            for (int u = 0; u < N; ++u) hsc[u] = sc[u];
            hp = p;
            hn = N;
        } else if (SC && active && head_lead) {
#pragma unroll
            for (int u = 0; u < N; ++u) {
                if constexpr (W32)
                    a.scores[(uint32_t)(p + u) * sc_edge + sc_lane] = sc[u];
                else
                    a.scores[(((int64_t)(p + u)) * B + b) * a.H + h] = sc[u];
            }
        }
        float mx = sc[0];
#pragma unroll
        for (int u = 1; u < N; ++u) mx = fmaxf(mx, sc[u]);
        if (fresh) {   // wave-uniform: the partial sums are still zero
            ms = mx;
            fresh = false;
        } else {
            const bool need = mx > ms + kLazy;
            if (__builtin_amdgcn_ballot_w64(need)) {
                // lanes that keep their reference scale by 1 (with a mask
                // their reference may still be -inf, and -inf - -inf is NaN)
                const float alpha = need ? fast_exp2(ms - mx) : 1.f;
                l *= alpha;
#pragma unroll
                for (int i = 0; i < CH; ++i) acc[i] *= alpha;
                ms = need ? mx : ms;
            }
        }
        // With a mask a lane may have seen no live key yet (ms = -inf); its
        // masked scores must then give weight 0, not exp2(-inf + inf).
        const float base = (KPM > 0 && ms == -INFINITY) ? 0.f : ms;
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const float pe = fast_exp2(sc[u] - base);
            l += pe;
            if constexpr (BF) {
                // The weight stays fp32: each bf16 value channel is widened
                // exactly (the low channel shifted up, the high one masked)
                // and multiplied in with a scalar fp32 fma.
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t w = vv[u].word(k);
                    acc[2 * k] = fmaf(pe, __uint_as_float(w << 16), acc[2 * k]);
                    acc[2 * k + 1] = fmaf(pe, __uint_as_float(w & 0xffff0000u), acc[2 * k + 1]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < CH; ++i) acc[i] = fmaf(pe, vv[u][i], acc[i]);
            }
        }
    }
};

template <typename T, int CH, int LPH, int U, int E_FUSE, bool QF, bool W32, bool SC, int KPM,
          int HOT = 0, bool COOP = false>
__global__ void __launch_bounds__(HOT ? 1024 : 256)
// (at least 7 wavefronts per SIMD: at most 72 VGPRs; the variants without the
// fused projections fit 64. The q-projecting variant without weights or mask
// fits 64 for 8 wavefronts once it stops prefetching the next piece's query
// chunk (below); with its prefetch it had needed 68, and squeezing that into
// 64 had spilled and run 5 % slower. With the hot-row cache one 16-wavefront
// workgroup fills a CU's LDS.)
__attribute__((amdgpu_waves_per_eu(HOT ? 4 : (QF && W32 && !SC && KPM == 0 ? 8 : 7))))
edge_fast(EdgeK a, const int32_t *__restrict__ csr_src, const int32_t *__restrict__ task_target,
          const int32_t *__restrict__ task_begin, const int32_t *__restrict__ task_end,
          const int32_t *__restrict__ task_slot, const uint32_t *__restrict__ kpm_csr)
{
    // The index arrays come in as noalias arguments: no store of this kernel
    // can reach them, so their wave-uniform reads stay scalar loads.
    static_assert(!QF || E_FUSE > 0, "the q prologue comes with the out_proj epilogue");
    static_assert(HOT == 0 || (QF && W32 && !SC && KPM == 0 && CH * sizeof(T) == 16),
                  "the hot-row cache serves the unmasked q-projecting kernel");
    static_assert(!COOP || (HOT == 0 && KPM == 0), "split targets merged here without a mask");
    constexpr int WPB = HOT ? 16 : 4;   // wavefronts per workgroup
    constexpr int WB = E_FUSE > 0 ? staged_bytes<T, E_FUSE>() : 16;
    __shared__ __attribute__((aligned(16))) char wlds[QF ? 2 * WB : WB];
    __shared__ __attribute__((aligned(16))) char hlds[HOT > 0 ? HOT * kHotSlot : 16];
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Split targets of at most 4 pieces can be merged here (COOP variants,
    // XCD-pinned launches only): the first coop_blocks workgroups each take
    // one (split target, sample group), wavefront w walks the target's piece
    // w, and after a workgroup barrier wavefront 0 merges the pieces in slot
    // order as merge_fast does, so no merge launch follows. Workgroup 8 r + x
    // serves split target r * xcd_per + x / passes for sample group
    // x % passes, on the XCDs that the main walk pins that group to; the main
    // walk numbers its workgroups from coop_blocks (a multiple of 8, so the
    // XCD of a number is unchanged) and skips the split pieces.
    const bool coop = COOP && blockIdx.x < a.coop_blocks;   // workgroup-uniform
    const uint32_t bid = COOP && !coop ? blockIdx.x - a.coop_blocks : blockIdx.x;
    // Each wavefront serves one sample group (pass) and walks the pieces
    // task0, task0 + tstride, ... (the host keeps n_tasks * passes below 2^31
    // and makes the wavefront count a multiple of passes).
    uint32_t task = 0, pass, coop_k = 0;
    if (coop) {
        const uint32_t x = bid & 7, xq = div31(x, a.pass_m, a.pass_sh);
        pass = x - xq * a.passes;
        coop_k = (bid >> 3) * a.xcd_per + xq;
    } else if (a.xcd_map == 1) {
        // Workgroups are dealt to the 8 XCDs round-robin; XCD x serves sample
        // group x % passes (passes divides 8), so its L2 caches only that
        // group's key/value rows.
        const uint32_t x = bid & 7, xq = div31(x, a.pass_m, a.pass_sh);
        pass = x - xq * a.passes;
        task = ((bid >> 3) * a.xcd_per + xq) * WPB + wave;
    } else if (a.xcd_map == 2) {
        // Sample groups one after another in launch order: the wavefronts in
        // flight read the key/value rows of few groups at a time.
        const uint32_t w = bid * WPB + wave;
        pass = div31(w, a.ts_m, a.ts_sh);
        task = w - pass * a.tstride;
    } else {
        const uint32_t w = bid * WPB + wave;
        task = div31(w, a.pass_m, a.pass_sh);
        pass = w - task * a.passes;
    }
    if constexpr (HOT > 0) {
        // The workgroup's sample group (pass: the same for all its wavefronts,
        // XCD-pinned launch) reads the key/value rows of a few popular
        // sources on a large share of its edges: their chunks are copied to
        // LDS once, in the lane order of the gathers, and read from there.
        constexpr int NF = HOT * (int)kHotSlot / 16 / (64 * WPB);   // chunks per thread
        static_assert(HOT * (int)kHotSlot / 16 % (64 * WPB) == 0, "whole chunks per thread");
        const int cpr = a.E / CH;
        uint4 v[NF];
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int f = threadIdx.x + 64 * WPB * i;
            const int slot = f >> 7, ln = f & 63;
            const uint32_t c = pass * 64 + ln;
            v[i] = make_uint4(0, 0, 0, 0);
            if (slot < a.n_hot && c < (uint32_t)(a.B * cpr)) {
                const int b = (int)div31(c, a.cpr_m, a.cpr_sh);
                const int col = ((int)c - b * cpr) * CH;
                uint64_t off = (uint64_t)a.hot_src[slot] * a.lay.kv_s + (uint64_t)b * a.lay.kv_b + col;
                if (f & 64)
                    off += a.lay.kv_v;
                v[i] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const T *>(a.kv) + off);
            }
        }
#pragma unroll
        for (int i = 0; i < NF; ++i)
            *reinterpret_cast<uint4 *>(hlds + (threadIdx.x + 64 * WPB * i) * 16) = v[i];
    }
    if constexpr (E_FUSE > 0) {
        // uniform over the launch; before any wavefront exits (the staging
        // is written for 256 threads)
        if (a.fuse_out && (HOT == 0 || threadIdx.x < 256)) {
            stage_wo<T, CH, E_FUSE>(a, wlds);
            if constexpr (QF)   // Wq after Wo
                stage_w<T, CH, E_FUSE>(a.wq, a.bq, wlds + WB);
        }
    }
    if (HOT > 0 || (E_FUSE > 0 && a.fuse_out))
        __syncthreads();
    if (coop ? coop_k >= (uint32_t)a.n_split : task >= (uint32_t)a.n_tasks)
        return;   // (workgroup-uniform for coop)

    // (held scores where they compile without spills: fp32, no fused
    // out_proj, no mask, heads of other than 2 lanes)
    EdgeLane<T, CH, LPH, W32, SC, KPM, (HOT > 0),
             (sizeof(T) == 4 && E_FUSE == 0 && KPM == 0 && LPH != 2)> st(a);
    st.src = csr_src;
    st.hl = hlds + lane * 16;
    const int B = a.B, E = a.E;
    const int cpr = E / CH;                       // chunks per sample row
    const uint32_t c = pass * 64 + lane;
    st.B = B;
    st.active = c < (uint32_t)(B * cpr);
    const int b = st.active ? (int)div31(c, a.cpr_m, a.cpr_sh) : 0;
    const int cr = (int)c - b * cpr;
    const int col = st.active ? cr * CH : 0;
    st.b = b;
    st.h = st.active ? cr / LPH : 0;
    st.head_lead = (lane % LPH) == 0;
    st.smul = a.scale;
    st.kbits = kpm_csr;
    st.kword = (pass * 64u / (uint32_t)cpr) >> 5;   // first sample of the pass / 32
    st.khi = ((uint32_t)b >> 5) != st.kword;         // (only KPM == 2 reads it)
    // byte offsets: per source (uniform), this lane's key and value chunks
    st.row2 = (uint64_t)a.lay.kv_s * sizeof(T);
    if constexpr (W32) {
        st.loff = ((uint32_t)b * (uint32_t)a.lay.kv_b + col) * (uint32_t)sizeof(T);
        st.vloff = st.loff + (uint32_t)a.lay.kv_v * (uint32_t)sizeof(T);
        st.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.kv), (short)0,
                                                    (int)(uint32_t)a.kv_bytes, 0x00020000);
        st.sc_edge = (uint32_t)(B * a.H);
        st.sc_lane = (uint32_t)b * a.H + st.h;
    } else {
        st.loff = (uint64_t)(b * a.lay.kv_b + col) * sizeof(T);
        st.vloff = st.loff + (uint64_t)a.lay.kv_v * sizeof(T);
    }
    st.kvb = reinterpret_cast<const char *>(a.kv);

    const T *qt = reinterpret_cast<const T *>(a.qt);
    auto load_q = [&](int tq) -> uint4 {
        const T *qa;
        if constexpr (W32)
            qa = qt + ((uint32_t)tq * (uint32_t)a.lay.q_t + (uint32_t)b * (uint32_t)a.lay.q_b + col);
        else
            qa = qt + tq * a.lay.q_t + b * a.lay.q_b + col;
        const uint4 *qp = reinterpret_cast<const uint4 *>(qa);
        return (a.nt & 1) ? load_nt(qp) : *qp;
    };

    // The next piece's query chunk is requested while this one runs, except
    // in the q-projecting kernel without weights or mask (32-bit offsets): there the four
    // registers it holds are what 8 wavefronts per SIMD need (63 registers,
    // no spills, against 72 and 7; gene edge kernel 128.5 -> 126.8 us).
    constexpr bool LEAN = QF && W32 && !SC && KPM == 0 && HOT == 0;
    uint4 qn = make_uint4(0, 0, 0, 0);
    // One piece of target t: its q (projected here with QF), the walk over
    // its edges, then its output row or, for a piece of a split target, its
    // partial; `mid` runs between the walk and the output.
    auto piece = [&](const int t, const int beg, const int end, const int slot, auto &&mid) {
        if constexpr (LEAN) {
            qn = load_q(t);
            st.q.u = q_proj_wave<T, CH, E_FUSE>(qn, lane, wlds + WB);
        } else if constexpr (QF) {
            st.q.u = q_proj_wave<T, CH, E_FUSE>(qn, lane, wlds + WB);
        } else {
            st.q.u = qn;
        }
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < CH; ++i) st.qf[i] = st.q[i] * a.scale;
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) st.acc[i] = 0.f;
        st.l = 0.f;
        st.ms = -INFINITY;
        st.fresh = true;

        static_assert(U == 4, "the tail below covers up to 3 edges");
        int p = beg;
        if constexpr (KPM == 0) {
            for (; p + U <= end; p += U)
                st.template step<U>(p);
        } else if (p + U <= end) {
            // full steps; each reads the next step's source ids in flight
            // (measured: pays with the mask's extra scalar loads, costs 2-5 %
            // without them)
            int cs[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cs[u] = csr_src[p + u];
            for (; p + 2 * U <= end; p += U) {
                st.template step<U, true>(p, cs);
#pragma unroll
                for (int u = 0; u < U; ++u) cs[u] = st.nsrc[u];
            }
            st.template step<U>(p, cs);
            p += U;
        }
        if (p + 2 <= end) {
            st.template step<2>(p);
            p += 2;
        }
        if (p < end)
            st.template step<1>(p);
        mid();
        st.flush_scores();
        const float m = st.ms, l = st.l;
        if (slot < 0) {
            const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
            float out[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) out[i] = st.acc[i] * inv;
            if (a.stat_ml && st.active && st.head_lead) {   // weights or training
                float *sp = a.stat_ml;
                if constexpr (W32)
                    sp += ((uint32_t)t * (uint32_t)B + (uint32_t)b) * (uint32_t)(2 * a.H) + 2 * st.h;
                else
                    sp += (((int64_t)t * B + b) * a.H + st.h) * 2;
                *reinterpret_cast<float2 *>(sp) = make_float2(m, l);
            }
            bool done = false;
            if constexpr (E_FUSE > 0) {
                if (a.fuse_out) {   // wave-uniform
                    out_proj_wave<T, CH, E_FUSE, W32>(a, out, lane, t, pass * (64 / (E_FUSE / CH)), wlds);
                    done = true;
                }
            }
            if (!done && st.active) {
                T *dst = reinterpret_cast<T *>(a.mixed);
                if constexpr (W32)
                    dst += (uint32_t)t * (uint32_t)a.lay.m_t + (uint32_t)b * (uint32_t)a.lay.m_b + col;
                else
                    dst += t * a.lay.m_t + b * a.lay.m_b + col;
                store_chunk<T, CH>(dst, out, (a.nt & 2) != 0);
            }
        } else if (st.active) {
            float *pa = a.part_acc, *pm = a.part_ml;
            if constexpr (W32) {
                pa += ((uint32_t)slot * (uint32_t)B + (uint32_t)b) * (uint32_t)E + col;
                pm += ((uint32_t)slot * (uint32_t)B + (uint32_t)b) * (uint32_t)(2 * a.H) + 2 * st.h;
            } else {
                pa += ((int64_t)slot * B + b) * E + col;
                pm += (((int64_t)slot * B + b) * a.H + st.h) * 2;
            }
            *reinterpret_cast<float4 *>(pa) = make_float4(st.acc[0], st.acc[1], st.acc[2], st.acc[3]);
            if constexpr (CH == 8)
                *reinterpret_cast<float4 *>(pa + 4) =
                    make_float4(st.acc[4], st.acc[5], st.acc[6], st.acc[7]);
            if (st.head_lead)
                *reinterpret_cast<float2 *>(pm) = make_float2(m, l);
        }
    };
    if constexpr (COOP) {
        if (coop) {
            // piece `wave` of the split target, cut as the index build cuts it
            const int cnt = a.split_count[coop_k];
            if ((int)wave < cnt) {   // wave-uniform
                const int t = a.split_target[coop_k];
                const int64_t r0 = a.row_ptr[t], g = a.row_ptr[t + 1] - r0;
                const int beg = (int)(r0 + ((int64_t)wave * g) / cnt);
                const int end = (int)(r0 + ((int64_t)(wave + 1) * g) / cnt);
                if constexpr (!LEAN)
                    qn = load_q(t);
                piece(t, beg, end, a.split_slot0[coop_k] + (int)wave, [] {});
            }
            // every wavefront of the workgroup gets here; the barrier orders
            // the pieces' partial stores before wavefront 0 reads them back
            __syncthreads();
            if (wave == 0)
                merge_split<T, CH, LPH, E_FUSE, 1>(a, coop_k, (int)pass, true, lane, wlds, [] {});
            return;
        }
    }
    int t = task_target[task];
    int beg = task_begin[task], end = task_end[task];
    int slot = task_slot[task];
    if constexpr (!LEAN)
        qn = load_q(t);
    for (;;) {
        // The next piece's bounds and query chunk are requested while this
        // one runs (wave-uniform branch).
        const uint32_t nxt = task + a.tstride;
        const bool more = nxt < (uint32_t)a.n_tasks;
        int t2 = 0, beg2 = 0, end2 = 0, slot2 = 0;
        if (more) {
            t2 = task_target[nxt];
            beg2 = task_begin[nxt];
            end2 = task_end[nxt];
            slot2 = task_slot[nxt];
        }
        auto next_q = [&] {
            if (!LEAN && more)
                qn = load_q(t2);
        };
        if (!COOP || slot < 0)   // (split pieces are the coop workgroups')
            piece(t, beg, end, slot, next_q);
        else
            next_q();
        if (!more)
            break;
        task = nxt;
        t = t2;
        beg = beg2;
        end = end2;
        slot = slot2;
    }
}

// Calibration (not part of the forward): the loads of edge_fast with no
// arithmetic beyond folding the loaded words together with XOR. The same
// grid, piece walk, lane layout and gather index: per piece the target's
// query chunk, per edge the source's key and value chunks (buffer loads with
// a uniform row offset, four edges in flight), and per piece one 16-byte
// store where edge_fast stores a mixed chunk. Its launch time is what the
// memory path takes for exactly edge_fast's access pattern.
template <typename T, int CH>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7)))
gather_probe(EdgeK a, const int32_t *__restrict__ csr_src, const int32_t *__restrict__ task_target,
             const int32_t *__restrict__ task_begin, const int32_t *__restrict__ task_end)
{
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
    constexpr int WPB = 4;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t task, pass;
    if (a.xcd_map == 1) {
        const uint32_t x = blockIdx.x & 7, xq = div31(x, a.pass_m, a.pass_sh);
        pass = x - xq * a.passes;
        task = ((blockIdx.x >> 3) * a.xcd_per + xq) * WPB + wave;
    } else if (a.xcd_map == 2) {
        const uint32_t w = blockIdx.x * WPB + wave;
        pass = div31(w, a.ts_m, a.ts_sh);
        task = w - pass * a.tstride;
    } else {
        const uint32_t w = blockIdx.x * WPB + wave;
        task = div31(w, a.pass_m, a.pass_sh);
        pass = w - task * a.passes;
    }
    if (task >= (uint32_t)a.n_tasks)
        return;
    const int cpr = a.E / CH;
    const uint32_t c = pass * 64 + lane;
    const bool active = c < (uint32_t)(a.B * cpr);
    const int b = active ? (int)div31(c, a.cpr_m, a.cpr_sh) : 0;
    const int col = active ? ((int)c - b * cpr) * CH : 0;
    const uint32_t row2 = (uint32_t)a.lay.kv_s * (uint32_t)sizeof(T);
    const uint32_t loff = ((uint32_t)b * (uint32_t)a.lay.kv_b + col) * (uint32_t)sizeof(T);
    const uint32_t vloff = loff + (uint32_t)a.lay.kv_v * (uint32_t)sizeof(T);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(a.kv), (short)0, (int)(uint32_t)a.kv_bytes, 0x00020000);
    const T *qt = reinterpret_cast<const T *>(a.qt);
    T *mixed = reinterpret_cast<T *>(a.mixed);
    for (;;) {
        const int t = task_target[task], beg = task_begin[task], end = task_end[task];
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            qt + ((uint32_t)t * (uint32_t)a.lay.q_t + (uint32_t)b * (uint32_t)a.lay.q_b + col));
        uint4 acc = (a.nt & 1) ? load_nt(qp) : *qp;
        int p = beg;
        for (; p + 4 <= end; p += 4) {
            u32x4 kw[4], vw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t so = (uint32_t)csr_src[p + u] * row2;
                kw[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, loff, so, 0);
                vw[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vloff, so, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc.x ^= kw[u].x ^ vw[u].x;
                acc.y ^= kw[u].y ^ vw[u].y;
                acc.z ^= kw[u].z ^ vw[u].z;
                acc.w ^= kw[u].w ^ vw[u].w;
            }
        }
        for (; p < end; ++p) {
            const uint32_t so = (uint32_t)csr_src[p] * row2;
            const u32x4 kw = __builtin_amdgcn_raw_buffer_load_b128(rsrc, loff, so, 0);
            const u32x4 vw = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vloff, so, 0);
            acc.x ^= kw.x ^ vw.x;
            acc.y ^= kw.y ^ vw.y;
            acc.z ^= kw.z ^ vw.z;
            acc.w ^= kw.w ^ vw.w;
        }
        if (active) {
            void *dst = mixed + ((uint32_t)t * (uint32_t)a.lay.m_t + (uint32_t)b * (uint32_t)a.lay.m_b + col);
            if (a.nt & 2)
                store_nt(dst, acc);
            else
                *reinterpret_cast<uint4 *>(dst) = acc;
        }
        task += a.tstride;
        if (task >= (uint32_t)a.n_tasks)
            break;
    }
}

// Any head size: one thread per (piece, sample, channel). Each thread forms
// the full dot product of its head on every edge.
template <typename T>
__global__ void __launch_bounds__(256) edge_generic(EdgeK a)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int B = a.B, E = a.E, d = a.d;
    const int64_t per_task = (int64_t)B * E;
    const int64_t task = idx / per_task;
    if (task >= a.n_tasks)
        return;
    const int rem = (int)(idx - task * per_task);
    const int b = rem / E, col = rem - b * E;
    const int h = col / d, c0 = h * d;
    const int t = a.task_target[task];
    const int beg = a.task_begin[task], end = a.task_end[task];
    const int slot = a.task_slot[task];
    const T *qt = reinterpret_cast<const T *>(a.qt) + t * a.lay.q_t + b * a.lay.q_b + c0;
    const T *kv = reinterpret_cast<const T *>(a.kv);
    const int64_t row2 = a.lay.kv_s, voff = a.lay.kv_v;
    auto ld = [](const T *p) -> float {
        if constexpr (sizeof(T) == 2) return bf2f(*p); else return *p;
    };
    float m = -INFINITY, l = 0.f, acc = 0.f;
    for (int p = beg; p < end; ++p) {
        if (a.kpm_bits &&   // key left out for this sample
            ((a.kpm_bits[(int64_t)a.orig_src[p] * a.kpm_words + (b >> 6)] >> (b & 63)) & 1u)) {
            if (a.scores && col == c0)
                a.scores[((int64_t)p * B + b) * a.H + h] = -INFINITY;
            continue;
        }
        const T *kr = kv + (int64_t)a.csr_src[p] * row2 + b * a.lay.kv_b + c0;
        float dot = 0.f;
        for (int i = 0; i < d; ++i) dot = fmaf(ld(qt + i) * a.scale, ld(kr + i), dot);
        if (a.scores && col == c0)
            a.scores[((int64_t)p * B + b) * a.H + h] = dot;
        const float mx = fmaxf(m, dot);
        const float alpha = fast_exp2(m - mx), pe = fast_exp2(dot - mx);
        l = l * alpha + pe;
        acc = fmaf(pe, ld(kr + voff + (col - c0)), acc * alpha);
        m = mx;
    }
    if (slot < 0) {
        const float o = l > 0.f ? acc / l : 0.f;
        T *dst = reinterpret_cast<T *>(a.mixed) + t * a.lay.m_t + b * a.lay.m_b + col;
        if constexpr (sizeof(T) == 2) *dst = f2bf(o); else *dst = o;
        if (a.stat_ml && col == c0) {
            float *st = a.stat_ml + (((int64_t)t * B + b) * a.H + h) * 2;
            st[0] = m;
            st[1] = l;
        }
    } else {
        a.part_acc[((int64_t)slot * B + b) * E + col] = acc;
        if (col == c0) {
            float *pm = a.part_ml + (((int64_t)slot * B + b) * a.H + h) * 2;
            pm[0] = m;
            pm[1] = l;
        }
    }
}

// Merge the pieces of each split target, in piece order. Same lane layout
// as edge_fast: one wavefront per (split target, sample group).
// The merge as a launch of its own: one wavefront per (split target, sample
// group).
template <typename T, int CH, int LPH, int E_FUSE>
__global__ void __launch_bounds__(256) merge_fast(EdgeK a)
{
    __shared__ __attribute__((aligned(16))) char wlds[E_FUSE > 0 ? staged_bytes<T, E_FUSE>() : 16];
    const int lane = threadIdx.x & 63;
    const uint32_t unit = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool valid = unit < (uint32_t)(a.n_split * a.passes);
    const uint32_t k = valid ? div31(unit, a.pass_m, a.pass_sh) : 0;
    const int pass = (int)(unit - k * a.passes);
    merge_split<T, CH, LPH, E_FUSE, 4>(a, k, pass, valid, lane, wlds, [&]() {
        if constexpr (E_FUSE > 0) {
            if (a.fuse_out) {   // (every wavefront of the workgroup takes part)
                stage_wo<T, CH, E_FUSE>(a, wlds);
                __syncthreads();
            }
        }
    });
}

// Any head size: one thread per (split target, sample, channel).
template <typename T>
__global__ void __launch_bounds__(256) merge_generic(EdgeK a)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int B = a.B, E = a.E;
    const int64_t per = (int64_t)B * E;
    const int64_t k = idx / per;
    if (k >= a.n_split)
        return;
    const int rem = (int)(idx - k * per);
    const int b = rem / E, col = rem - b * E, h = col / a.d;
    const int t = a.split_target[k], s0 = a.split_slot0[k], n = a.split_count[k];
    float M = -INFINITY;
    for (int j = 0; j < n; ++j)
        M = fmaxf(M, a.part_ml[(((int64_t)(s0 + j) * B + b) * a.H + h) * 2]);
    float l = 0.f, acc = 0.f;
    for (int j = 0; j < n; ++j) {
        const float *pm = a.part_ml + (((int64_t)(s0 + j) * B + b) * a.H + h) * 2;
        const float w = pm[1] > 0.f ? fast_exp2(pm[0] - M) : 0.f;
        l = fmaf(pm[1], w, l);
        acc = fmaf(a.part_acc[((int64_t)(s0 + j) * B + b) * E + col], w, acc);
    }
    const float o = l > 0.f ? acc / l : 0.f;
    T *dst = reinterpret_cast<T *>(a.mixed) + t * a.lay.m_t + b * a.lay.m_b + col;
    if constexpr (sizeof(T) == 2) *dst = f2bf(o); else *dst = o;
    if (a.stat_ml && col == h * a.d) {
        float *st = a.stat_ml + (((int64_t)t * B + b) * a.H + h) * 2;
        st[0] = M;
        st[1] = l;
    }
}

// need_weights: weight = exp2(score - max) / sum, written in edge order.
// A workgroup takes 64 consecutive CSR positions for every sample: pairs
// (position, sample) with the sample fastest read the stored scores and the
// targets' (max, sum) contiguously; head-averaged weights then go through LDS
// so that each sample's row is written with the position fastest (edges of
// one target sit together in the edge order as well as in the CSR).
constexpr int kWeightTile = 64;      // CSR positions per workgroup
constexpr int kWeightSamples = 256;  // samples per workgroup (blockIdx.y: sample chunk)

__device__ inline float edge_weight(float sc, float m, float l)
{
    return l > 0.f ? fast_exp2(sc - m) / l : 0.f;   // l = 0: every key of the target masked
}

// The H weights of one (edge, sample): scores sc[h], statistics st[2h] (max)
// and st[2h + 1] (sum); 16-byte loads when H is a multiple of 4.
template <typename F> __device__ inline void head_weights(const float *sc, const float *st, int H, F &&f)
{
    if ((H & 3) == 0) {
        for (int h = 0; h < H; h += 4) {
            const float4 s4 = *reinterpret_cast<const float4 *>(sc + h);
            const float4 a = *reinterpret_cast<const float4 *>(st + 2 * h);
            const float4 b = *reinterpret_cast<const float4 *>(st + 2 * h + 4);
            f(h, edge_weight(s4.x, a.x, a.y));
            f(h + 1, edge_weight(s4.y, a.z, a.w));
            f(h + 2, edge_weight(s4.z, b.x, b.y));
            f(h + 3, edge_weight(s4.w, b.z, b.w));
        }
    } else {
        for (int h = 0; h < H; ++h)
            f(h, edge_weight(sc[h], st[2 * h], st[2 * h + 1]));
    }
}

// HC: the head count as a constant (its loops unrolled, loads batched), or 0.
template <int HC>
__global__ void __launch_bounds__(256) weights_kernel(EdgeK a)
{
    extern __shared__ float wt[];   // [samples of the chunk][kWeightTile] head averages
    const int B = a.B, H = HC > 0 ? HC : a.H;
    const int64_t p0 = (int64_t)blockIdx.x * kWeightTile;
    const int b0 = blockIdx.y * kWeightSamples;
    const int np = (int)(a.nnz - p0 < kWeightTile ? a.nnz - p0 : kWeightTile);
    const int nb = B - b0 < kWeightSamples ? B - b0 : kWeightSamples;
    const int n = np * nb;
    if (!a.average) {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int pl = i / nb, bl = i - pl * nb, b = b0 + bl;
            const int64_t p = p0 + pl;
            const int t = a.csr_tgt[p];
            const float *sc = a.scores + (p * B + b) * H;
            const float *st = a.stat_ml + ((int64_t)t * B + b) * H * 2;
            float *w = a.weights + ((int64_t)b * a.nnz + a.csr_eid[p]) * H;
            head_weights(sc, st, H, [&](int h, float v) { w[h] = v; });
        }
        return;
    }
    // Averaged: KB pairs per thread at a time, every load of the KB pairs
    // issued before any is used (indices past the end re-read the last pair;
    // only the LDS stores are guarded).
    constexpr int KB = 4;
    for (int i0 = threadIdx.x; i0 < n; i0 += KB * blockDim.x) {
        int pl[KB], bl[KB], t[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int i = min(i0 + k * (int)blockDim.x, n - 1);
            pl[k] = i / nb;
            bl[k] = i - pl[k] * nb;
            t[k] = a.csr_tgt[p0 + pl[k]];
        }
        float v[KB];
        if constexpr (HC > 0 && HC % 4 == 0) {
            // every pair's scores and statistics as 16-byte loads, then the sums
            float4 s4[KB][HC / 4], m4[KB][HC / 2];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int b = b0 + bl[k];
                const float4 *sc = reinterpret_cast<const float4 *>(a.scores + ((p0 + pl[k]) * B + b) * HC);
                const float4 *st = reinterpret_cast<const float4 *>(a.stat_ml + ((int64_t)t[k] * B + b) * HC * 2);
#pragma unroll
                for (int j = 0; j < HC / 4; ++j) s4[k][j] = sc[j];
#pragma unroll
                for (int j = 0; j < HC / 2; ++j) m4[k][j] = st[j];
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                float sum = 0.f;
#pragma unroll
                for (int j = 0; j < HC / 4; ++j) {
                    const float4 a0 = m4[k][2 * j], a1 = m4[k][2 * j + 1];
                    sum += edge_weight(s4[k][j].x, a0.x, a0.y);
                    sum += edge_weight(s4[k][j].y, a0.z, a0.w);
                    sum += edge_weight(s4[k][j].z, a1.x, a1.y);
                    sum += edge_weight(s4[k][j].w, a1.z, a1.w);
                }
                v[k] = sum / (float)HC;
            }
        } else {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int b = b0 + bl[k];
                const float *sc = a.scores + ((p0 + pl[k]) * B + b) * H;
                const float *st = a.stat_ml + ((int64_t)t[k] * B + b) * H * 2;
                float sum = 0.f;
                head_weights(sc, st, H, [&](int, float w) { sum += w; });
                v[k] = sum / (float)H;
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            if (i0 + k * (int)blockDim.x < n)
                wt[bl[k] * kWeightTile + pl[k]] = v[k];
        }
    }
    __syncthreads();
    // each sample's weights in edge order (positions fastest), KB at a time
    for (int i0 = threadIdx.x; i0 < n; i0 += KB * blockDim.x) {
        int e[KB], bl[KB], pl[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int i = min(i0 + k * (int)blockDim.x, n - 1);
            bl[k] = i / np;
            pl[k] = i - bl[k] * np;
            e[k] = a.csr_eid[p0 + pl[k]];
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            if (i0 + k * (int)blockDim.x < n)
                a.weights[(int64_t)(b0 + bl[k]) * a.nnz + e[k]] = wt[bl[k] * kWeightTile + pl[k]];
        }
    }
}

// Multiplier and shift with floor(n / d) = (n * m) >> sh for 0 <= n < 2^31
// and 1 <= d < 2^31: l = ceil(log2 d), m = floor(2^(31 + l) / d) + 1 < 2^32,
// sh = 31 + l (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, with N = 31).
void magic31(uint32_t d, uint32_t &m, int &sh)
{
    int l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    m = (uint32_t)((((uint64_t)1 << (31 + l)) / d) + 1);
    sh = 31 + l;
}

void set_passes(EdgeK &k, int ch)
{
    const int64_t chunks = (int64_t)k.B * (k.E / ch);
    k.passes = (int)((chunks + 63) / 64);
    magic31((uint32_t)k.passes, k.pass_m, k.pass_sh);
    magic31((uint32_t)(k.E / ch), k.cpr_m, k.cpr_sh);
}

// Whether every tensor the edge kernel addresses is under 2 GiB (then it
// uses 32-bit offsets).
bool offsets32(const EdgeK &k, size_t es)
{
    const uint64_t rows = (uint64_t)k.L * k.B * k.E * es;
    const uint64_t scores = k.scores ? (uint64_t)k.nnz * k.B * k.H * 4 : 0;
    const uint64_t parts = (uint64_t)k.n_slots * k.B * k.E * 4;
    const uint64_t stats = (uint64_t)k.L * k.B * k.H * 8;
    const uint64_t lim = (uint64_t)1 << 31;
    return k.kv_bytes < lim && rows < lim && scores < lim && parts < lim && stats < lim;
}

EdgeK make_k(const EdgeArgs &x)
{
    EdgeK k{};   // fields a launch does not set stay zero
    const GraphDev *g = x.g;
    k.csr_src = x.gather_src;   // key/value workspace rows
    k.csr_tgt = g->csr_tgt;
    k.csr_eid = g->csr_eid;
    k.task_target = g->task_target;
    k.task_begin = g->task_begin;
    k.task_end = g->task_end;
    k.task_slot = g->task_slot;
    k.split_target = g->split_target;
    k.split_slot0 = g->split_slot0;
    k.split_count = g->split_count;
    k.n_tasks = g->n_tasks;
    k.n_split = g->n_split;
    k.n_slots = g->n_slots;
    k.B = (int)x.B;
    k.E = (int)x.E;
    k.H = (int)x.H;
    k.d = (int)(x.E / x.H);
    k.nnz = x.nnz;
    k.passes = 1;
    k.xcd_map = x.xcd_map;
    k.tstride = 0;
    k.kpm_bits = x.kpm_bits;
    k.kpm_csr = x.kpm_csr;
    k.kpm_w32 = x.kpm_w32;
    k.kpm_words = x.kpm_words;
    k.orig_src = g->csr_src;
    k.nt = x.nt;
    k.fuse_out = x.fuse_out;
    k.L = (int)x.L;
    k.wo = x.wo;
    k.bo = x.bo;
    k.fuse_in = x.fuse_in;
    k.wq = x.wq;
    k.bq = x.bq;
    k.out = x.out;
    k.scale = (float)(1.4426950408889634 / sqrt((double)k.d));
    k.lay = x.lay;
    k.kv_bytes = x.kv_bytes;
    k.qt = x.qt;
    k.kv = x.kv;
    k.mixed = x.mixed;
    k.part_acc = x.part_acc;
    k.part_ml = x.part_ml;
    k.stat_ml = x.stat_ml;
    k.scores = x.scores;
    k.weights = x.weights;
    k.average = x.average;
    k.hot_src = x.hot_src;
    k.hot_csr = x.hot_csr;
    k.n_hot = x.hot_csr && x.hot_src ? x.n_hot : 0;
    k.row_ptr = g->row_ptr;
    k.allow_coop = x.coop && x.max_pieces <= 4 && !x.hot_csr;
    k.coop_blocks = 0;
    return k;
}

// Whether a launch of edge_fast with these (passes set) merges the split
// targets itself: each has at most 4 pieces, the sample groups are pinned to
// XCDs and there is no mask (the launch also needs 32-bit offsets).
bool coop_merge(const EdgeK &k)
{
    return k.allow_coop && k.n_split > 0 && k.xcd_map == 1 && 8 % k.passes == 0 && !k.kpm_bits;
}

int cu_count()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    if (dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Workgroup count of an edge_fast launch of wpb wavefronts per workgroup and
// at most cap workgroups, and the walk it implies: sets k.xcd_map (the
// order actually used), xcd_per, tstride and its divisor. (The gather probe
// takes the same grid, so that it walks the pieces in the same order.)
int64_t edge_grid(EdgeK &k, int wpb, int64_t cap)
{
    int64_t blocks;
    if (k.xcd_map == 1 && 8 % k.passes == 0) {
        const int64_t per = 8 / k.passes;   // workgroups per pass per round of 8
        int64_t rounds = (k.n_tasks + wpb * per - 1) / (wpb * per);
        rounds = std::min(rounds, std::max<int64_t>(1, cap / 8));
        blocks = 8 * rounds;
        k.xcd_per = (uint32_t)per;
        k.tstride = (uint32_t)(rounds * per * wpb);
    } else {
        if (k.xcd_map != 2 || k.passes == 1)
            k.xcd_map = 0;
        // whole multiples of `passes` wavefronts, so each keeps its pass
        const int64_t g = k.passes / std::__gcd<int64_t>(4, k.passes);
        blocks = (k.n_tasks * k.passes + 3) / 4;
        blocks = std::min(blocks, std::max<int64_t>(g, cap));
        blocks = (blocks + g - 1) / g * g;
        k.tstride = (uint32_t)(blocks * 4 / k.passes);
        magic31(k.tstride, k.ts_m, k.ts_sh);
    }
    return blocks;
}

template <typename T, int CH, int LPH, int E_FUSE, bool QF>
hipError_t run_fast(EdgeK k, int persist, hipStream_t s)
{
    set_passes(k, CH);
    if (k.n_tasks * k.passes >= ((int64_t)1 << 31))
        return hipErrorInvalidConfiguration;
    // Workgroups of 4 wavefronts. With persist > 0 at most persist
    // workgroups per CU are launched and each wavefront walks several
    // pieces; otherwise one wavefront per (piece, sample group).
    const bool w32 = offsets32(k, sizeof(T));
    // Hot-row cache: one resident 16-wavefront workgroup per CU, XCD-pinned
    // sample groups (each workgroup serves one group).
    constexpr int kHot = kHotRows;
    const bool hot = QF && k.n_hot > 0 && k.n_hot <= kHot && k.xcd_map == 1 &&
                     8 % k.passes == 0 && w32 && !k.scores && !k.kpm_bits;
    const int wpb = hot ? 16 : 4;
    const int64_t cap = hot ? (int64_t)cu_count()
                            : persist > 0 ? (int64_t)cu_count() * persist : ((int64_t)1 << 40);
    unsigned nb = (unsigned)edge_grid(k, wpb, cap);
    if (!hot && w32 && coop_merge(k)) {   // (edge_grid keeps xcd_map 1 only where pinned)
        k.coop_blocks = (uint32_t)(8 * ((k.n_split + k.xcd_per - 1) / k.xcd_per));
        nb += k.coop_blocks;
    }
    if constexpr (QF) {
        if (hot) {
            edge_fast<T, CH, LPH, 4, E_FUSE, QF, true, false, 0, kHot><<<nb, 1024, 0, s>>>(
                k, k.hot_csr, k.task_target, k.task_begin, k.task_end, k.task_slot, k.kpm_csr);
            return hipGetLastError();
        }
    }
#define PMA_EDGE_LAUNCH(W, S, M)                                                          \
    edge_fast<T, CH, LPH, 4, E_FUSE, QF, W, S, M><<<nb, 256, 0, s>>>(                    \
        k, k.csr_src, k.task_target, k.task_begin, k.task_end, k.task_slot, k.kpm_csr)
    if (k.coop_blocks > 0) {   // (coop_merge: no mask, 32-bit offsets)
        if (k.scores)
            edge_fast<T, CH, LPH, 4, E_FUSE, QF, true, true, 0, 0, true><<<nb, 256, 0, s>>>(
                k, k.csr_src, k.task_target, k.task_begin, k.task_end, k.task_slot, k.kpm_csr);
        else
            edge_fast<T, CH, LPH, 4, E_FUSE, QF, true, false, 0, 0, true><<<nb, 256, 0, s>>>(
                k, k.csr_src, k.task_target, k.task_begin, k.task_end, k.task_slot, k.kpm_csr);
        return hipGetLastError();
    }
    if (k.kpm_bits) {
        if (!k.kpm_csr)
            return hipErrorInvalidValue;
        if (!w32)   // refused by mask_supported()
            return hipErrorInvalidValue;
        // One 32-bit word per position holds a wavefront's samples when the
        // chunks per row are a power of two of at least 2 (then a wavefront
        // covers 64 / cpr <= 32 samples starting at a multiple of 64 / cpr).
        // Otherwise (64 samples per wavefront, or e.g. 3 heads of one chunk:
        // wavefronts of 21-22 samples starting anywhere) its samples may
        // straddle two words.
        const int cpr = k.E / CH;
        if (cpr == 1 || (cpr & (cpr - 1)) != 0) {
            if constexpr (E_FUSE == 0) {   // (embed_dim 64 has 8 or 16 chunks per row)
                if (k.scores)
                    PMA_EDGE_LAUNCH(true, true, 2);
                else
                    PMA_EDGE_LAUNCH(true, false, 2);
            } else {
                return hipErrorInvalidValue;
            }
        } else if (k.scores) {
            PMA_EDGE_LAUNCH(true, true, 1);
        } else {
            PMA_EDGE_LAUNCH(true, false, 1);
        }
    } else if (w32 && k.scores)
        PMA_EDGE_LAUNCH(true, true, 0);
    else if (w32)
        PMA_EDGE_LAUNCH(true, false, 0);
    else if (k.scores)
        PMA_EDGE_LAUNCH(false, true, 0);
    else
        PMA_EDGE_LAUNCH(false, false, 0);
#undef PMA_EDGE_LAUNCH
    return hipGetLastError();
}

// out_proj can run in the edge kernel's epilogue when a wavefront holds at
// least 4 samples' rows (E / CH <= 16 chunks per row); it is used for E = 64
// (out_fusable).
template <typename T, int CH>
constexpr bool fusable(int E)
{
    return E == 64 && E / CH <= 16;
}

template <typename T, int CH, int LPH>
hipError_t run_fast_any(EdgeK k, int persist, hipStream_t s)
{
    const bool ok = k.fuse_out && k.E == 64 && fusable<T, CH>(64);
    if (k.fuse_in) {   // q exists only in the prologue: no way back
        // (bf16 only: an fp32 Wq beside Wo is 33 KB of LDS per workgroup,
        // too much for the gather's occupancy; refused by q_fusable)
        if constexpr (sizeof(T) == 2) {
            if (ok)
                return run_fast<T, CH, LPH, 64, true>(k, persist, s);
        }
        return hipErrorInvalidValue;
    }
    if (ok)
        return run_fast<T, CH, LPH, 64, false>(k, persist, s);
    k.fuse_out = 0;
    return run_fast<T, CH, LPH, 0, false>(k, persist, s);
}

template <typename T>
hipError_t dispatch_edge(EdgeK k, int persist, hipStream_t s)
{
    constexpr int CH = 16 / sizeof(T);
    if (k.d % CH == 0) {
        switch (k.d / CH) {
        case 1: return run_fast_any<T, CH, 1>(k, persist, s);
        case 2: return run_fast_any<T, CH, 2>(k, persist, s);
        case 4: return run_fast_any<T, CH, 4>(k, persist, s);
        case 8: return run_fast_any<T, CH, 8>(k, persist, s);
        case 16: return run_fast_any<T, CH, 16>(k, persist, s);
        default: break;
        }
    }
    if (k.fuse_in)   // refused by the host (out_fusable)
        return hipErrorInvalidValue;
    const int64_t n = k.n_tasks * k.B * k.E;
    edge_generic<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(k);
    return hipGetLastError();
}

template <typename T, int CH, int LPH>
hipError_t run_merge(EdgeK k, hipStream_t s)
{
    set_passes(k, CH);
    const int64_t units = k.n_split * k.passes;
    if (units >= ((int64_t)1 << 31))
        return hipErrorInvalidConfiguration;
    const unsigned blocks = (unsigned)((units + 3) / 4);
    if (k.fuse_out && k.E == 64 && fusable<T, CH>(64)) {
        merge_fast<T, CH, LPH, 64><<<blocks, 256, 0, s>>>(k);
    } else {
        k.fuse_out = 0;
        merge_fast<T, CH, LPH, 0><<<blocks, 256, 0, s>>>(k);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_merge(EdgeK k, hipStream_t s)
{
    constexpr int CH = 16 / sizeof(T);
    if (k.d % CH == 0) {
        switch (k.d / CH) {
        case 1: return run_merge<T, CH, 1>(k, s);
        case 2: return run_merge<T, CH, 2>(k, s);
        case 4: return run_merge<T, CH, 4>(k, s);
        case 8: return run_merge<T, CH, 8>(k, s);
        case 16: return run_merge<T, CH, 16>(k, s);
        default: break;
        }
    }
    const int64_t n = k.n_split * k.B * k.E;
    merge_generic<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(k);
    return hipGetLastError();
}

// key_padding_mask bytes -> bits by source: thread (s, w) gathers samples
// 64 w .. 64 w + 63 of key s (reads of consecutive s are coalesced).
__global__ void pack_mask_kernel(const uint8_t *mask, int64_t bstride, int64_t B, int64_t S,
                                 int words, uint64_t *bits)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= S * words)
        return;
    const int64_t w = i / S, s = i - w * S;
    const int nb = (int)(B - w * 64 < 64 ? B - w * 64 : 64);
    // all 64 loads independent (samples past B re-read the last one and are
    // dropped), so they are in flight together
    uint64_t v = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
        const int64_t b = w * 64 + (j < nb ? j : nb - 1);
        const uint64_t m = mask[b * bstride + s] != 0 && j < nb;
        v |= m << j;
    }
    bits[s * words + w] = v;
}

// The packed bits in CSR order, as 32-bit words:
// out[p * w32 + j] = half j % 2 of bits[src[p] * words + j / 2].
__global__ void gather_mask_kernel(const uint64_t *bits, int words, int w32, const int32_t *src,
                                   int64_t nnz, uint32_t *out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nnz * w32)
        return;
    const int64_t p = i / w32;
    const int j = (int)(i - p * w32);
    out[i] = (uint32_t)(bits[(int64_t)src[p] * words + j / 2] >> (32 * (j & 1)));
}

}  // namespace

pma_status pack_mask(const uint8_t *mask, int64_t bstride, int64_t B, int64_t S, uint64_t *bits,
                     hipStream_t s)
{
    const int words = (int)((B + 63) / 64);
    const int64_t n = S * words;
    pack_mask_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(mask, bstride, B, S, words, bits);
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status gather_mask(const uint64_t *bits, int words, int w32, const int32_t *src, int64_t nnz,
                       uint32_t *out, hipStream_t s)
{
    const int64_t n = nnz * w32;
    if (n == 0)
        return PMA_OK;
    gather_mask_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(bits, words, w32, src, nnz, out);
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

bool mask_supported(const EdgeArgs &x)
{
    // the per-position mask words are indexed with 32 bits
    if ((uint64_t)x.nnz * (uint64_t)((x.B + 31) / 32) >= ((uint64_t)1 << 31))
        return false;
    const EdgeK k = make_k(x);
    const int64_t ch = x.dt == PMA_BF16 ? 8 : 4, d = x.E / x.H;
    const bool fast = d % ch == 0 && (d / ch) <= 16 && ((d / ch) & (d / ch - 1)) == 0;
    return !fast || offsets32(k, x.dt == PMA_BF16 ? 2 : 4);
}

bool out_fusable(int64_t E, int64_t H, pma_dtype dt)
{
    // E = 128 would stage a 32 KB Wo per 4-wavefront workgroup, which halves
    // the gather's occupancy; measured, the separate out_proj is faster there.
    const int64_t d = E / H;
    const int64_t ch = dt == PMA_BF16 ? 8 : 4;
    return E == 64 && d % ch == 0 && (d / ch) <= 16 && ((d / ch) & (d / ch - 1)) == 0;
}

bool q_fusable(int64_t E, int64_t H, pma_dtype dt)
{
    return dt == PMA_BF16 && out_fusable(E, H, dt);
}

Layout make_layout(bool batch_first, int64_t B, int64_t L, int64_t S, int64_t E)
{
    Layout y;
    if (batch_first) {
        y.q_t = E;
        y.q_b = L * E;
        y.kv_s = E;
        y.kv_b = S * E;
        y.kv_v = B * S * E;
        y.m_t = E;
        y.m_b = L * E;
    } else {
        y.q_t = B * E;
        y.q_b = E;
        y.kv_s = 2 * B * E;
        y.kv_b = E;
        y.kv_v = B * E;
        y.m_t = B * E;
        y.m_b = E;
    }
    return y;
}

bool edge_merges_splits(const EdgeArgs &x)
{
    EdgeK k = make_k(x);
    const int ch = x.dt == PMA_BF16 ? 8 : 4;
    if (k.d % ch != 0)
        return false;   // the per-channel kernel: merge launch
    const int lph = k.d / ch;
    if (lph > 16 || (lph & (lph - 1)) != 0)
        return false;
    set_passes(k, ch);
    return coop_merge(k) && offsets32(k, x.dt == PMA_BF16 ? 2 : 4);
}

pma_status launch_edge(const EdgeArgs &x, hipStream_t s)
{
    EdgeK k = make_k(x);
    hipError_t e = x.dt == PMA_BF16 ? dispatch_edge<uint16_t>(k, x.persist, s)
                                    : dispatch_edge<float>(k, x.persist, s);
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status launch_gather_probe(const EdgeArgs &x, hipStream_t s)
{
    EdgeK k = make_k(x);
    const size_t es = x.dt == PMA_BF16 ? 2 : 4;
    const int ch = (int)(16 / es);
    const int64_t lph = k.d % ch == 0 ? k.d / ch : 0;
    if (lph < 1 || lph > 16 || (lph & (lph - 1)) != 0)
        return PMA_E_UNSUPPORTED;   // head sizes of the per-channel kernel
    set_passes(k, ch);
    if (k.n_tasks * k.passes >= ((int64_t)1 << 31) || !offsets32(k, es))
        return PMA_E_UNSUPPORTED;
    const int64_t cap = x.persist > 0 ? (int64_t)cu_count() * x.persist : ((int64_t)1 << 40);
    const unsigned nb = (unsigned)edge_grid(k, 4, cap);
    if (x.dt == PMA_BF16)
        gather_probe<uint16_t, 8><<<nb, 256, 0, s>>>(k, k.csr_src, k.task_target, k.task_begin,
                                                     k.task_end);
    else
        gather_probe<float, 4><<<nb, 256, 0, s>>>(k, k.csr_src, k.task_target, k.task_begin,
                                                  k.task_end);
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status launch_merge(const EdgeArgs &x, hipStream_t s)
{
    EdgeK k = make_k(x);
    if (k.n_split == 0)
        return PMA_OK;
    hipError_t e = x.dt == PMA_BF16 ? dispatch_merge<uint16_t>(k, s) : dispatch_merge<float>(k, s);
    return e == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

pma_status launch_weights(const EdgeArgs &x, hipStream_t s)
{
    EdgeK k = make_k(x);
    const int64_t chunk_b = k.B < kWeightSamples ? k.B : kWeightSamples;
    const size_t lds = x.average ? (size_t)chunk_b * kWeightTile * sizeof(float) : 0;
    const dim3 g((unsigned)((k.nnz + kWeightTile - 1) / kWeightTile),
                 (unsigned)((k.B + kWeightSamples - 1) / kWeightSamples));
    switch (k.average ? k.H : 0) {   // (per-head weights: the plain loop)
    case 1: weights_kernel<1><<<g, 256, lds, s>>>(k); break;
    case 2: weights_kernel<2><<<g, 256, lds, s>>>(k); break;
    case 4: weights_kernel<4><<<g, 256, lds, s>>>(k); break;
    case 8: weights_kernel<8><<<g, 256, lds, s>>>(k); break;
    case 16: weights_kernel<16><<<g, 256, lds, s>>>(k); break;
    default: weights_kernel<0><<<g, 256, lds, s>>>(k); break;
    }
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
