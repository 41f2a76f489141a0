// Host-side part of the C ABI: status strings, buffer sizes and the weight
// codec (ternary rows -> W_nonzero / W_negative bitplanes, "BitState / HSDR
// PoC Technical Brief - v0.5", section 4; 128-weight groups with one integer
// scale, "A standalone deterministic integer inference engine for
// BitNet-style LLMs", sections 4.2-4.3; the BITNET_PLANES eight-plane rows of
// "[bitnet] T2: lm_head via BITNET_PLANES weight format").
//
// The codec runs once at load time, on the host, synchronously.
#include <string.h>

#include <vector>

#include "bs_internal.h"

using namespace bs;

extern "C" int32_t bs_abi_version(void) { return BS_ABI_VERSION; }

extern "C" const char *bs_status_str(int32_t status) {
    switch (status) {
    case BS_OK: return "ok";
    case BS_E_NULL: return "null pointer argument";
    case BS_E_SHAPE: return "invalid shape (sizes must be positive, k a multiple of 128)";
    case BS_E_RANGE: return "argument value out of range";
    case BS_E_OVERFLOW: return "shape breaks the static integer overflow bound";
    case BS_E_HIP: return "HIP runtime or kernel launch error";
    case BS_E_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case BS_E_ALIGN: return "device pointer not aligned as documented";
    default: return "unknown status";
    }
}

static int32_t codec_shape(int64_t rows, int64_t k) {
    if (rows < 1 || k < kGroup || k % kGroup != 0) return BS_E_SHAPE;
    return BS_OK;
}

extern "C" int64_t bs_ternary_planes_bytes(int64_t rows, int64_t k) {
    int32_t st = codec_shape(rows, k);
    return st ? st : pad64(rows) * k / 4;
}

extern "C" int64_t bs_ternary_scales_count(int64_t rows, int64_t k) {
    int32_t st = codec_shape(rows, k);
    return st ? st : pad64(rows) * (k / kGroup);
}

// Build the two 128-bit masks of one group of 128 trits.  Returns false on a
// value outside {-1, 0, +1}.
static bool group_masks(const int8_t *t, uint8_t nz[16], uint8_t neg[16]) {
    memset(nz, 0, 16);
    memset(neg, 0, 16);
    for (int i = 0; i < 128; ++i) {
        int8_t w = t[i];
        if (w == 0) continue;
        if (w != 1 && w != -1) return false;
        nz[i >> 3] |= (uint8_t)(1u << (i & 7));
        if (w < 0) neg[i >> 3] |= (uint8_t)(1u << (i & 7));
    }
    return true;
}

extern "C" int32_t bs_ternary_pack(const int8_t *t, int64_t rows, int64_t k, uint8_t *planes) {
    if (!t || !planes) return BS_E_NULL;
    if (int32_t st = codec_shape(rows, k)) return st;
    const int64_t G = k / kGroup, R = pad64(rows);
    memset(planes, 0, (size_t)(R * k / 4));
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t tile = r / kTileRows, j = r % kTileRows;
        for (int64_t g = 0; g < G; ++g) {
            uint8_t *blk = planes + (tile * G + g) * 2048;
            if (!group_masks(t + r * k + g * kGroup, blk + 16 * j, blk + 1024 + 16 * j))
                return BS_E_RANGE;
        }
    }
    return BS_OK;
}

extern "C" int32_t bs_ternary_unpack(const uint8_t *planes, int64_t rows, int64_t k, int8_t *t) {
    if (!t || !planes) return BS_E_NULL;
    if (int32_t st = codec_shape(rows, k)) return st;
    const int64_t G = k / kGroup;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t tile = r / kTileRows, j = r % kTileRows;
        for (int64_t g = 0; g < G; ++g) {
            const uint8_t *nz = planes + (tile * G + g) * 2048 + 16 * j;
            const uint8_t *neg = nz + 1024;
            for (int i = 0; i < 128; ++i) {
                int a = (nz[i >> 3] >> (i & 7)) & 1, b = (neg[i >> 3] >> (i & 7)) & 1;
                if (b && !a) return BS_E_RANGE;
                t[r * k + g * kGroup + i] = (int8_t)(a ? (b ? -1 : 1) : 0);
            }
        }
    }
    return BS_OK;
}

extern "C" int32_t bs_ternary_pack_scales(const int16_t *scales, int64_t rows, int64_t k,
                                          int16_t *packed) {
    if (!scales || !packed) return BS_E_NULL;
    if (int32_t st = codec_shape(rows, k)) return st;
    const int64_t G = k / kGroup, R = pad64(rows);
    memset(packed, 0, (size_t)(R * G) * sizeof(int16_t));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < G; ++g)
            packed[((r / kScaleRows) * G + g) * kScaleRows + r % kScaleRows] = scales[r * G + g];
    return BS_OK;
}

extern "C" int64_t bs_q1_planes_bytes(int64_t rows, int64_t k) {
    int32_t st = codec_shape(rows, k);
    return st ? st : pad64(rows) * k / 8;
}

// One sign bit per weight (1 = +1) in the tiled layout of one ternary plane.
extern "C" int32_t bs_q1_pack(const int8_t *signs, int64_t rows, int64_t k, uint8_t *bits) {
    if (!signs || !bits) return BS_E_NULL;
    if (int32_t st = codec_shape(rows, k)) return st;
    const int64_t G = k / kGroup, R = pad64(rows);
    memset(bits, 0, (size_t)(R * k / 8));
    for (int64_t r = 0; r < rows; ++r) {
        const int8_t *row = signs + r * k;
        for (int64_t g = 0; g < G; ++g) {
            uint8_t *f = bits + ((r / kTileRows) * G + g) * 1024 + 16 * (r % kTileRows);
            for (int i = 0; i < 128; ++i) {
                const int8_t v = row[g * kGroup + i];
                if (v == 1) f[i >> 3] |= (uint8_t)(1u << (i & 7));
                else if (v != -1) return BS_E_RANGE;
            }
        }
    }
    return BS_OK;
}

extern "C" int64_t bs_planes03_bytes(int64_t vocab, int64_t dim) {
    int32_t st = codec_shape(vocab, dim);
    return st ? st : pad64(vocab) * dim;
}

extern "C" int64_t bs_planes47_bytes(int64_t vocab, int64_t dim) {
    int32_t st = codec_shape(vocab, dim);
    return st ? st : vocab * dim;
}

// Planes 0-3 and 4-7 of a position are stored as their balanced-ternary
// digit sums (27, 9, 3, 1 weights): one int8 in [-40, 40] per position for
// each half, which keeps the four trits and costs the same byte as four pairs
// of bitplane bits.  The half read by the full-vocabulary scan is tiled in
// 16-position runs (run c of row j of a 64-row tile at 1024c + 16j of the
// tile's 8192-byte group block); the other half is row major.
extern "C" int32_t bs_planes_pack(const int8_t *trits, int64_t vocab, int64_t dim,
                                  uint8_t *planes03, uint8_t *planes47) {
    if (!trits || !planes03 || !planes47) return BS_E_NULL;
    if (int32_t st = codec_shape(vocab, dim)) return st;
    const int64_t G = dim / kGroup, R = pad64(vocab);
    memset(planes03, 0, (size_t)(R * dim));
    std::vector<int8_t> hi((size_t)dim);
    for (int64_t r = 0; r < vocab; ++r) {
        const int8_t *tr = trits + r * 8 * dim;
        int8_t *lo = reinterpret_cast<int8_t *>(planes47 + r * dim);
        for (int64_t i = 0; i < dim; ++i) {
            int a = 0, b = 0;
            for (int q = 0; q < 4; ++q) {
                const int8_t u = tr[q * dim + i], v = tr[(q + 4) * dim + i];
                if (u < -1 || u > 1 || v < -1 || v > 1) return BS_E_RANGE;
                a = 3 * a + u;
                b = 3 * b + v;
            }
            hi[(size_t)i] = (int8_t)a;
            lo[i] = (int8_t)b;
        }
        const int64_t tile = r / kTileRows, j = r % kTileRows;
        for (int64_t g = 0; g < G; ++g)
            for (int c = 0; c < 8; ++c)
                memcpy(planes03 + (tile * G + g) * 8192 + 1024 * c + 16 * j,
                       hi.data() + g * kGroup + 16 * c, 16);
    }
    return BS_OK;
}
