// Calibration of the memory path (not part of the method): random-row
// gathers at the edge kernel's lane layout, from a table of any size, so that
// the edge kernel's gathers can be read against what each level of the
// memory hierarchy delivers for them (pma_gather_ceiling in include/pma.h).
#include "pma_internal.h"

namespace pma {
namespace {

// Calibration (not part of the forward): wavefronts gather whole 1 KB rows
// of a table, one 16-byte chunk per lane, at the row indices rows[0 .. n):
// wavefront w takes rows w per .. w per + per - 1, eight in flight, folding
// the loaded words together with XOR, and stores one 16-byte word per lane at
// the end. With the table sized to stay in L1, in L2, in the last-level
// cache or only in HBM, its rate is what the vector memory path delivers for
// such gathers from that level. The row offset is uniform (a scalar operand
// of the buffer load); a row index past the table is clamped to its last row.
__global__ void __launch_bounds__(256)
gather_ceiling(const void *table, uint32_t table_bytes, const int32_t *__restrict__ rows, int64_t n,
               int per, uint4 *sink)
{
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const uint32_t w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t beg = (int64_t)w * per;
    if (beg >= n)
        return;
    const int64_t end = beg + per < n ? beg + per : n;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(table), (short)0, (int)table_bytes, 0x00020000);
    const uint32_t lo = (uint32_t)lane * 16, last = (table_bytes >> 10) - 1;
    auto row = [&](int64_t j) -> uint32_t {   // uniform
        const uint32_t r = (uint32_t)rows[j];
        return (r < last ? r : last) << 10;
    };
    u32x4 acc = {0, 0, 0, 0};
    int64_t i = beg;
    for (; i + U <= end; i += U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lo, row(i + u), 0);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < end; ++i)
        acc ^= __builtin_amdgcn_raw_buffer_load_b128(rs, lo, row(i), 0);
    sink[(uint64_t)w * 64 + lane] = make_uint4(acc.x, acc.y, acc.z, acc.w);
}

}  // namespace

pma_status launch_gather_ceiling(const void *table, uint64_t table_bytes, const int32_t *rows,
                                 int64_t n, int64_t per, void *sink, hipStream_t s)
{
    const int64_t waves = (n + per - 1) / per;
    const int64_t blocks = (waves + 3) / 4;
    gather_ceiling<<<(unsigned)blocks, 256, 0, s>>>(table, (uint32_t)table_bytes, rows, n, (int)per,
                                                    reinterpret_cast<uint4 *>(sink));
    return hipGetLastError() == hipSuccess ? PMA_OK : PMA_E_DEVICE;
}

}  // namespace pma
