// gemm_common.hpp -- pieces shared by the gfx950 MFMA GEMMs of libqproj.
//
// Tiling: a 256-thread workgroup (4 waves in a 2x2 arrangement) owns a
// BM x BN output tile; each wave owns a (BM/2) x (BN/2) sub-tile made of
// 32x32 MFMA tiles.  K advances in stages of BKB bytes per row; both operand
// tiles of a stage are staged in LDS (double-buffered, one barrier per
// stage) with 16 bytes of padding per row against bank conflicts.
//
// Tile order: see tile_coords (banded M-fast order, XCD-contiguous).
#pragma once

#include "qp_device.hpp"

namespace qp {

// MFMA 32x32 output layout (16 accumulator registers per lane): register r
// of lane l holds row 8*(r/4) + 4*(l/32) + (r%4) and column l%32.
__device__ __forceinline__ int mfma32_row(int r, int lane)
{
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Map a workgroup to its (m-tile, n-tile).  Tiles are numbered in bands of
// GROUP_M m-tiles: inside a band the m-tile index runs fastest and the band
// then walks across n (the M-fast order w4a4_gemm_mfast uses, confined to a
// band).  The linear workgroup id is first remapped so that each XCD runs a
// contiguous range of that order; its ~32 resident workgroups then cover an
// 8 x 4 block of tiles whose operand stages fit in the XCD's L2, instead of
// one weight panel against every activation tile.
constexpr uint32_t GROUP_M = 8;

// Tile at position id of the banded order.
__device__ __forceinline__ void banded_tile(uint32_t id, uint32_t mtiles, uint32_t ntiles,
                                            uint32_t &tm, uint32_t &tn)
{
    uint32_t per_band = GROUP_M * ntiles;
    uint32_t band = id / per_band, rem = id % per_band;
    uint32_t band_m0 = band * GROUP_M;
    uint32_t rows = mtiles - band_m0 < GROUP_M ? mtiles - band_m0 : GROUP_M;
    tm = band_m0 + rem % rows;
    tn = rem / rows;
}

// Tile of linear workgroup id v.
__device__ __forceinline__ void tile_coords_of(uint32_t v, uint32_t mtiles, uint32_t ntiles,
                                               uint32_t &tm, uint32_t &tn)
{
    banded_tile(xcd_remap(v, mtiles * ntiles), mtiles, ntiles, tm, tn);
}

__device__ __forceinline__ void tile_coords(uint32_t mtiles, uint32_t ntiles,
                                            uint32_t &tm, uint32_t &tn)
{
    tile_coords_of(blockIdx.x, mtiles, ntiles, tm, tn);
}

// Tile orders a launch may ask for (the tile-order ablation): 0 = the banded,
// XCD-aware order above; 1 = plain M-fast (workgroup id = tm + mtiles * tn,
// consecutive workgroups share a weight panel); 2 = plain N-fast (consecutive
// workgroups share an activation panel).
// Tile at position id of order 0 (banded, without the XCD remap), 1 or 2.
__device__ __forceinline__ void tile_in_order(uint32_t order, uint32_t id, uint32_t mtiles,
                                              uint32_t ntiles, uint32_t &tm, uint32_t &tn)
{
    if (order == 1) {
        tm = id % mtiles;
        tn = id / mtiles;
    } else if (order == 2) {
        tn = id % ntiles;
        tm = id / ntiles;
    } else {
        banded_tile(id, mtiles, ntiles, tm, tn);
    }
}

__device__ __forceinline__ void tile_coords_order(uint32_t order, uint32_t mtiles,
                                                  uint32_t ntiles, uint32_t &tm, uint32_t &tn)
{
    if (order == 1) {
        tm = blockIdx.x % mtiles;
        tn = blockIdx.x / mtiles;
    } else if (order == 2) {
        tn = blockIdx.x % ntiles;
        tm = blockIdx.x / ntiles;
    } else {
        tile_coords(mtiles, ntiles, tm, tn);
    }
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

// ---------------------------------------------------------------------------
// Large-tile machinery (256 x 256 workgroup tiles, stages of 128 bytes of K
// per operand row).
//
// Operand stages go global -> LDS with 16-byte LDS-DMA loads
// (global_load_lds_dwordx4): no register staging, so two stages in flight
// cost no VGPRs.  One 64-lane DMA instruction fills 1 KB of LDS = 8 rows x
// 128 bytes; lane i lands at byte 16*i of that kilobyte, i.e. row i/8,
// physical chunk i%8.  Rows are unpadded and the eight 16-byte chunks of row
// r are stored XOR-swizzled (logical chunk c at physical c ^ ((r/2) % 8)).
// An MFMA fragment read has 16 consecutive rows fetch one logical chunk; the
// 64 banks span two 128-byte rows, so rows of equal parity share a bank half
// and the swizzle gives each of them a different 16-byte slot within it.
// Each lane simply fetches the logical chunk that belongs in its physical
// slot.
// ---------------------------------------------------------------------------
constexpr int BIG_ROWS = 256;     // rows per operand stage
constexpr int BIG_KB = 128;       // bytes of K per row per stage

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// DMA one operand stage: rows row0 .. row0+255 (clamped to nrows-1), bytes
// k0 .. k0+127 of each row (row stride ld), into the 32 KB at lds.
// Every wave issues 8 instructions; wave w fills kilobytes 8w .. 8w+7.
__device__ __forceinline__ void dma_stage(const uint8_t *__restrict__ base, size_t ld,
                                          uint32_t row0, uint32_t nrows, uint32_t k0,
                                          uint8_t *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r_in = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int kb = 8 * wave + j;                      // kilobyte index 0..31
        int row = 8 * kb + r_in;                    // tile row 0..255
        uint32_t gr = row0 + row;
        gr = gr < nrows ? gr : nrows - 1;
        const uint8_t *src = base + (size_t)gr * ld + k0 + 16 * swz(row, slot);
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds + 1024 * kb), 16, 0, 0);
    }
}

// Read logical 16-byte chunk c of tile row `row` from a swizzled stage.
__device__ __forceinline__ u32x4 lds_chunk(const uint8_t *lds, int row, int c)
{
    return *reinterpret_cast<const u32x4 *>(lds + row * BIG_KB + 16 * swz(row, c));
}

// s_waitcnt immediate that waits for vmcnt <= n and for lgkmcnt == 0, and
// not for expcnt (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in bits 15:14).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

} // namespace qp
