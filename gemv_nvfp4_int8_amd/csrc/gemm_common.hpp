// gemm_common.hpp -- pieces shared by the gfx950 MFMA GEMMs of libqproj.
//
// Tiling: a 256-thread workgroup (4 waves in a 2x2 arrangement) owns a
// BM x BN output tile; each wave owns a (BM/2) x (BN/2) sub-tile made of
// 32x32 MFMA tiles.  K advances in stages of BKB bytes per row; both operand
// tiles of a stage are staged in LDS (double-buffered, one barrier per
// stage) with 16 bytes of padding per row against bank conflicts.
//
// Tile order: tiles are numbered M-fast (consecutive workgroups walk down M
// and share one weight panel, the grid order gemm_fp4.rs chooses for
// w4a4_gemm_mfast), and the linear id is remapped so that the tiles an XCD
// runs are contiguous in that order (each XCD has its own L2).
#pragma once

#include "qp_device.hpp"

namespace qp {

// MFMA 32x32 output layout (16 accumulator registers per lane): register r
// of lane l holds row 8*(r/4) + 4*(l/32) + (r%4) and column l%32.
__device__ __forceinline__ int mfma32_row(int r, int lane)
{
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Map a workgroup to its (m-tile, n-tile).
__device__ __forceinline__ void tile_coords(uint32_t mtiles, uint32_t ntiles,
                                            uint32_t &tm, uint32_t &tn)
{
    uint32_t total = mtiles * ntiles;
    uint32_t id = xcd_remap(blockIdx.x, total);
    tm = id % mtiles;
    tn = id / mtiles;
}

// Cooperative predicated copy of a ROWS x BKB-byte operand stage from global
// memory (row stride ld bytes) into registers: 16-byte chunks, chunk c of
// thread t is c = t + 256*j.  Rows >= nrows or columns >= kbytes load zero.
template <int ROWS, int BKB>
struct StageLoader {
    static constexpr int CHUNKS_PER_ROW = BKB / 16;
    static constexpr int PER_THREAD = ROWS * CHUNKS_PER_ROW / 256;
    static_assert(ROWS * CHUNKS_PER_ROW % 256 == 0, "stage must split evenly");
    u32x4 r[PER_THREAD];

    __device__ __forceinline__ void load(const uint8_t *__restrict__ base,
                                         size_t ld, uint32_t row0, uint32_t nrows,
                                         uint32_t k0, uint32_t kbytes)
    {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            int c = threadIdx.x + 256 * j;
            int row = c / CHUNKS_PER_ROW, kc = c % CHUNKS_PER_ROW;
            uint32_t gr = row0 + row, gk = k0 + 16u * kc;
            r[j] = (u32x4){0, 0, 0, 0};
            if (gr < nrows && gk < kbytes)
                r[j] = *reinterpret_cast<const u32x4 *>(base + (size_t)gr * ld + gk);
        }
    }

    // LDS layout: row-major with a pitch of BKB + 16 bytes.
    __device__ __forceinline__ void store(uint8_t *lds) const
    {
#pragma unroll
        for (int j = 0; j < PER_THREAD; ++j) {
            int c = threadIdx.x + 256 * j;
            int row = c / CHUNKS_PER_ROW, kc = c % CHUNKS_PER_ROW;
            *reinterpret_cast<u32x4 *>(lds + row * (BKB + 16) + 16 * kc) = r[j];
        }
    }
};

} // namespace qp
