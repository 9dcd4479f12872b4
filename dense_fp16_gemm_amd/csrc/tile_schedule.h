// Tile order of the persistent GEMM kernel, shared verbatim by the device
// code and by the host-side entry point the CPU tests call.
//
// Two layers:
//  1. Grouped rasterization (Tilus tutorial "Hopper matmul", page
//     "4. Pipeline Abstraction and Two Consumer Warp Groups", section Tile
//     Rasterization): the N axis of the tile grid is cut into groups of
//     `swizzle` tile columns; inside a group, linear ids walk the group's
//     tiles row by row (m outer, n inner); when tiles_n is not a multiple of
//     `swizzle` the last group is narrower, so the map stays a bijection.
//     Tiles that run together then share a few B column strips and A row
//     strips, which is what keeps B (and A) in cache.
//  2. XCD-aware slot order (gfx950-specific, not on the pages): the
//     persistent kernel's workgroup `wg` handles slots wg, wg + grid, ...
//     (page "6. Register Reallocation, Multicast, and a Persistent Kernel",
//     Persistent Tile Loop), and the dispatcher places workgroup `wg` on
//     XCD `wg % xcds`.  Each XCD has its own L2, so within one round we
//     hand each XCD a contiguous run of the round's linear ids; the raster
//     group then makes that run a compact block of tiles.  A round of n
//     active slots (n = grid, or fewer in a partial last round; any n, not
//     only multiples of xcds) gives XCD x the n / xcds ids after those of
//     XCDs 0..x-1, plus one more when x < n % xcds: exactly the number of
//     its workgroups below n, so the map is a bijection on [0, tiles).
#ifndef GEMM_F16_TILE_SCHEDULE_H
#define GEMM_F16_TILE_SCHEDULE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define GEMM_F16_HD __host__ __device__
#else
#define GEMM_F16_HD
#endif

namespace gemm_f16 {

// Linear tile id -> (tile_m, tile_n) with raster groups `swizzle` columns wide.
// Every argument is non-negative; the arithmetic is unsigned, which spares
// the device code the sign handling of signed division.
GEMM_F16_HD inline void grouped_tile(int32_t linear, int32_t tiles_m, int32_t tiles_n,
                                     int32_t swizzle, int32_t &tile_m, int32_t &tile_n)
{
    const uint32_t sw = static_cast<uint32_t>(swizzle);
    const uint32_t per_group = static_cast<uint32_t>(tiles_m) * sw;
    const uint32_t lin = static_cast<uint32_t>(linear);
    const uint32_t group = lin / per_group;
    const uint32_t in_group = lin - group * per_group;
    const uint32_t first_n = group * sw;
    const uint32_t rest = static_cast<uint32_t>(tiles_n) - first_n;
    const uint32_t width = rest < sw ? rest : sw;
    const uint32_t tm = in_group / width;
    tile_m = static_cast<int32_t>(tm);
    tile_n = static_cast<int32_t>(first_n + (in_group - tm * width));
}

// Persistent slot (round * grid + wg) -> linear tile id, XCD-contiguous.
GEMM_F16_HD inline int32_t slot_to_linear(int32_t slot, int32_t grid, int32_t tiles,
                                          int32_t xcds)
{
    if (xcds <= 1) return slot;
    const uint32_t g = static_cast<uint32_t>(grid), xc = static_cast<uint32_t>(xcds);
    const uint32_t sl = static_cast<uint32_t>(slot);
    const uint32_t round = sl / g;
    const uint32_t wg = sl - round * g;
    const uint32_t base = round * g;
    const uint32_t left = static_cast<uint32_t>(tiles) - base;
    const uint32_t n = left < g ? left : g;
    const uint32_t q = n / xc;
    const uint32_t r = n - q * xc;
    const uint32_t x = wg % xc;
    return static_cast<int32_t>(base + x * q + (x < r ? x : r) + wg / xc);
}

}  // namespace gemm_f16

#endif  // GEMM_F16_TILE_SCHEDULE_H
