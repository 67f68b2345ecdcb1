// Stream-K work split of the attention kernel (also checked on the host).
//
// Tiles are query tiles (128 or 256 rows) ordered (batch, head) major, query tile minor.
// With S resident workgroup slots (two per CU, or one for 256-row tiles), the first
// floor(tiles / S) * S tiles (n_dp of them) are taken whole by S persistent workgroups,
// in XCD-contiguous order so that the workgroups of one XCD share a head's K/V in L2.  When the remaining tiles are few (at
// most S/4) and long (at least 64 key blocks) they would leave most of the GPU idle in a
// last round for a long time, so their work is split evenly over G_sk workgroups of a
// second launch ("stream-K", plan_stream_k): W units, a unit being one 64-key block of one
// tile, and split workgroup g takes the contiguous units [g*q + min(g, r), +q + (g < r))
// with q = W / G_sk, r = W % G_sk.  (A grid of fewer tiles than half the slots, such as a
// Ring chunk of 1152 queries x 1152 keys, is not split: measured, pieces of 9 key blocks
// ran 1.3x slower than whole tiles.)  Such a range is processed as its pieces of
// consecutive tiles:
//   whole tile                      -> final O and LSE
//   piece starting inside a tile    -> the raw state (accumulators, reference max, row
//     (only a range's first piece)     sum per lane) goes to workspace slot g, then flag[g]
//                                      is set to this launch's flag value
//   piece starting a tile, ending   -> the tile's finaliser: after its own keys it waits
//     inside it (a range's last)       (bounded) for the flags of the workgroups that own
//                                      the rest of the tile, folds in their states and
//                                      writes O and LSE.
// A finaliser only waits for workgroups that need nothing from anyone before publishing,
// but nothing guarantees that they are resident at the same time: the workgroup ids are
// remapped to XCD-contiguous ranges, so a helper can be dispatched after its finaliser,
// and another stream or process can hold the compute units it would need.  The wait is
// therefore bounded (max_polls polls of the flags): if a flag does not carry the launch's
// value in time, the finaliser computes the rest of the tile itself.  The result never
// depends on timing and every wave terminates.
// The flag value of a launch mixes two counts, so that no flag left in the workspace by
// another launch matches it and the workspace never needs clearing: `epoch`, a host count
// of the library's split launches (unique per launch), and the word at `launch_ctr` in the
// workspace, which every workgroup reads at its start and a one-thread kernel enqueued
// after the split launch advances.  The second count makes replays of one captured launch
// (a HIP graph, whose host arguments are frozen) differ from each other as well.
#pragma once

#include <hip/hip_runtime.h>

namespace dtl {

struct StreamK {
    int n_dp;                   // whole-tile workgroups (tiles [0, n_dp))
    int n_kv;                   // units (64-key blocks) per tile
    int G_sk;                   // split workgroups (0: none)
    long q;                     // split part: units per workgroup (W / G_sk)
    int r;                      // split part: workgroups with one unit more (W % G_sk)
    float* ws_acc;              // [G_sk][waves][D/8 stores][64 lanes][4] accumulators
    float* ws_ml;               // [G_sk][threads][4] reference max, row-sum half, 2 unused
    unsigned long long* flag;   // [G_sk]
    unsigned long long epoch;   // host count of split launches (see the flag value above)
    unsigned long long* launch_ctr;   // workspace word advanced after every split launch
    int slots;                  // resident workgroups the schedule assumes (whole-tile grid bound)
    int max_polls;              // a finaliser's bound on polls of its helpers' flags (0: none)
};

// The flag value of a split launch: its host count mixed with the workspace's launch count.
__host__ __device__ __forceinline__ unsigned long long sk_flag_value(unsigned long long epoch,
                                                                     unsigned long long launches) {
    return epoch ^ (launches * 0x9E3779B97F4A7C15ull);
}

// First unit of split-part workgroup g (g = G_sk gives W).
__host__ __device__ __forceinline__ long sk_first_unit(const StreamK& w, int g) {
    return (long)g * w.q + (g < w.r ? g : w.r);
}

// The schedule for `tiles` tiles of n_kv key blocks on `slots` workgroup slots: whole
// tiles [0, n_dp), the rest split over G_sk workgroups (none when G_sk = 0).
// force: -1 the rule above, 0 never split, 1 split any remainder of at least two key blocks
__host__ __device__ inline StreamK plan_stream_k(long tiles, int n_kv, long slots, int force = -1) {
    StreamK w = {};
    w.n_kv = n_kv;
    const long rem = tiles % slots;
    const bool split = tiles >= slots && rem > 0 &&
                       (force < 0 ? rem * 4 <= slots && n_kv >= 64 : force == 1 && n_kv >= 2);
    w.n_dp = (int)(split ? tiles - rem : tiles);   // a multiple of the slot count when split
    const long W = (tiles - w.n_dp) * n_kv;        // units of the split part
    w.G_sk = (int)(W < slots ? W : slots);
    if (w.G_sk > 0) {
        w.q = W / w.G_sk;
        w.r = (int)(W % w.G_sk);
    }
    return w;
}

// Workgroup that owns unit u < W.
__host__ __device__ __forceinline__ int sk_owner(const StreamK& w, long u) {
    const long big = (long)w.r * (w.q + 1);
    return u < big ? (int)(u / (w.q + 1)) : w.r + (int)((u - big) / w.q);
}

}  // namespace dtl
