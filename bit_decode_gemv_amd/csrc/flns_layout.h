// Table blob of the pure fractional-LNS reduction (internal to the library).
//
//   bytes [0, 64)      int32 header: magic, frac_bits, n_kp, n_km, bytes per
//                      correction entry (2 or 4), total bytes, stride S, 0...
//   bytes [64, 592)    int32 fold table fold[n] = round(N*log2 n), n = 0..128
//                      (fold[0] = 0 is never used; 132 slots keep 16-byte
//                      alignment)
//   bytes [592, ...)   corrections in two runs of S = max(n_kp, n_km) + 1
//                      entries: same-sign kp[D] at D, opposite-sign km[D] at
//                      S + D (km[0] unused), every slot past a table's end
//                      zero, so an index clamped to S - 1 reads a zero
//                      correction; int16 for frac_bits <= 8 (every value
//                      fits), int32 above; padded to 16 bytes.
#pragma once

#include <stdint.h>

namespace bs {

constexpr int32_t kFlnsMagic = 0x534E4C46;
constexpr int64_t kFlnsHdrBytes = 64;
constexpr int64_t kFlnsFoldSlots = 132;
constexpr int64_t kFlnsCorrOff = kFlnsHdrBytes + kFlnsFoldSlots * 4;
constexpr int kFlnsSmallMaxFrac = 8;
// 2 * S at frac_bits = 8 (S = 25661), the largest int16 table, rounded up
// to a multiple of 8 entries.
constexpr int kFlnsSmallMaxEntries = 51328;

struct FlnsSizes {
    int64_t n_kp, n_km, stride, elem, bytes;
};

// Table lengths and blob size for frac_bits f (host; false if f is out of
// range).
bool flns_sizes(int f, FlnsSizes *s);

// round(8*2^f * log2 d) for d >= 1; false if this host cannot round it
// unambiguously.
bool flns_log_scale(int f, uint32_t d, int64_t *out);

}  // namespace bs
