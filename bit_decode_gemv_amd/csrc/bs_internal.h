// Internal declarations shared by the host-side C-ABI code and the kernel
// launchers of the library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "bs.h"

namespace bs {

constexpr int64_t kGroup = 128;      // weights per scale group
constexpr int64_t kTileRows = 64;    // rows per tile = lanes per wavefront
constexpr int64_t kScaleRows = 16;   // rows per block of the packed scales
constexpr size_t kWsAlign = 256;     // workspace alignment

inline int64_t pad64(int64_t rows) { return (rows + 63) / 64 * 64; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape checks shared by the entry points.
inline int32_t check_rows_k(int64_t rows, int64_t k, int64_t k_max) {
    if (rows < 1 || k < kGroup || k % kGroup != 0) return BS_E_SHAPE;
    // the kernels index rows (and the last tile's padding rows) in int32
    if (rows > ((int64_t)1 << 31) - 64) return BS_E_SHAPE;
    if (k > k_max) return BS_E_OVERFLOW;
    return BS_OK;
}

inline bool ws_ok(const void *ws, size_t have, size_t need) {
    return ws != nullptr && have >= need && ((uintptr_t)ws % kWsAlign) == 0;
}

// Split-K geometry of a tiled GEMV: each workgroup covers one 64-row tile
// and `gpb` consecutive 128-weight groups; `nsplit` workgroups share a tile.
struct SplitK {
    int64_t tiles;
    int64_t groups;
    int64_t gpb;
    int64_t nsplit;
};

inline SplitK plan_splitk(int64_t rows, int64_t k, int64_t target_wgs) {
    SplitK s;
    s.tiles = pad64(rows) / kTileRows;
    s.groups = k / kGroup;
    int64_t want = (target_wgs + s.tiles - 1) / s.tiles;
    if (want < 1) want = 1;
    if (want > s.groups) want = s.groups;
    s.gpb = (s.groups + want - 1) / want;
    s.nsplit = (s.groups + s.gpb - 1) / s.gpb;
    return s;
}

}  // namespace bs
