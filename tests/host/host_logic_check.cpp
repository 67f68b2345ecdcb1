// Host-side checks of the index helpers the kernels use (built with hipcc, run on the CPU).
//   fastdiv: FastDiv::div(n) == n / d for edge and random n, many d
//   xcd:     xcd_contiguous is a bijection on [0, total) for many totals
//   streamk: the attention's unit ranges partition [0, W) into G near-equal ranges and
//            sk_owner inverts them; the schedule (plan_stream_k) splits only a short last round
//   runmap:  for the three permutes and many shapes, RunMap::source agrees with the
//            element index map written out directly, stays in bounds and is a bijection
//   tile:    the attention's LDS key-tile layout (head_dim 64 and 128, 4- and 8-wave
//            workgroups): the direct loads
//            fill every row and chunk of a tile once, the K and V^T fragment reads (the
//            latter through the transposing read's lane exchange) return exactly the
//            elements the MFMA operands need, and no read has a bank conflict
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <vector>

#include "common.h"
#include "fastdiv.h"
#include "runmap.h"
#include "streamk.h"
#include "tile_layout.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // xorshift64*
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (uint32_t)((rng * 2685821657736338717ull) >> 32);
}

// A tile in LDS as (key, 16-byte chunk) per 16-byte slot, filled by the load placement.
template <int D, int NW>
static long check_tile_layout() {
    using L = dtl::TileLayout<D, NW>;
    long bad = 0;
    auto fail = [&](const char* what, int a, int b, int c) {
        if (bad < 10) printf("tile D=%d NW=%d %s %d %d %d\n", D, NW, what, a, b, c);
        ++bad;
    };
    for (int tensor = 0; tensor < 2; ++tensor) {
        const int slots = L::kTileBytes / 16;
        std::vector<int> key_at(slots, -1), chunk_at(slots, -1), seen(slots, 0);
        for (int w = 0; w < NW; ++w)
            for (int i = 0; i < L::kLoadsPerWave; ++i)
                for (int l = 0; l < 64; ++l) {
                    const int byte = L::load_block(w, i) + 16 * l;
                    if (byte != L::load_row(w, i, l) * L::kRowBytes + 16 * (l % L::kChunks)) fail("block", w, i, l);
                    const int key = tensor ? L::v_src_key(w, i, l) : L::k_src_key(w, i, l);
                    const int ch = tensor ? L::v_src_chunk(w, i, l) : L::k_src_chunk(w, i, l);
                    if (byte < 0 || byte >= L::kTileBytes || key < 0 || key >= 64 || ch < 0 || ch >= L::kChunks) {
                        fail("range", w, i, l);
                        continue;
                    }
                    key_at[byte / 16] = key; chunk_at[byte / 16] = ch;
                    ++seen[key * L::kChunks + ch];
                }
        for (int e = 0; e < slots; ++e)
            if (seen[e] != 1) fail("fill", tensor, e, seen[e]);
        if (tensor == 0) {
            // The S^T = K Q^T accumulator of a 32x32 MFMA holds, in register i of lane l, output
            // row 8 (i/4) + 4 (l/32) + i%4 (the A row, i.e. the LDS row within the key half);
            // with the rows permuted by krow_slot that is key 16 (i/8) + 8 (l/32) + i%8, the
            // order in which the P.V product takes its B operand.
            for (int l = 0; l < 64; ++l)
                for (int i = 0; i < 16; ++i)
                    if (dtl::krow_slot(8 * (i / 4) + 4 * (l / 32) + i % 4) != 16 * (i / 8) + 8 * (l / 32) + i % 8)
                        fail("kperm", l, i, 0);
            // K: lane l of read (kb, ks) gets chunk 2 ks + l/32 of key krow_slot(kb*32 + l%32)
            for (int kb = 0; kb < 2; ++kb)
                for (int ks = 0; ks < D / 16; ++ks) {
                    std::vector<int> bank_used(16 * 4, 0);
                    for (int l = 0; l < 64; ++l) {
                        const int off = L::k_frag(kb, ks, l);
                        if (off % 16 || off < 0 || off >= L::kTileBytes) { fail("kread", kb, ks, l); continue; }
                        if (key_at[off / 16] != dtl::krow_slot(kb * 32 + (l & 31)) || chunk_at[off / 16] != 2 * ks + (l >> 5))
                            fail("kfrag", kb, ks, l);
                        // 16 lanes (256 bytes) per LDS cycle: their 16-byte bank groups must differ
                        if (bank_used[(l / 16) * 16 + (off / 16) % 16]++) fail("kbank", kb, ks, l);
                    }
                }
        } else {
            // V^T: the transposing read gives lane l (in its 16-lane group G) element l%4 of
            // the 8 bytes that lane 16G + 4 rho + (l%16)/4 addressed, for rho = 0..3; that must
            // be V[key kb*32 + hf*16 + 8 (l/32) + 4 j + rho][column db*32 + l%32].
            for (int kb = 0; kb < 2; ++kb)
                for (int hf = 0; hf < 2; ++hf)
                    for (int db = 0; db < D / 32; ++db)
                        for (int j = 0; j < 2; ++j) {
                            std::vector<int> bank_used(32 * 2, 0);
                            for (int l = 0; l < 64; ++l) {
                                const int off = L::v_frag(kb, hf, db, j, l);
                                if (off % 8 || off < 0 || off >= L::kTileBytes) { fail("vread", kb, hf, l); continue; }
                                // 32 lanes x 8 bytes per LDS cycle: distinct 8-byte bank pairs
                                if (bank_used[(l / 32) * 32 + (off / 8) % 32]++) fail("vbank", kb, db, l);
                            }
                            for (int l = 0; l < 64; ++l) {
                                const int G = l / 16;
                                for (int rho = 0; rho < 4; ++rho) {
                                    const int src_lane = 16 * G + 4 * rho + (l % 16) / 4;
                                    const int off = L::v_frag(kb, hf, db, j, src_lane) + 2 * (l % 4);
                                    const int key = key_at[off / 16];
                                    const int col = 8 * chunk_at[off / 16] + (off % 16) / 2;
                                    if (key != kb * 32 + hf * 16 + 8 * (l >> 5) + 4 * j + rho || col != db * 32 + (l & 31))
                                        fail("vfrag", kb * 4 + hf * 2 + j, db, l);
                                }
                            }
                        }
        }
    }
    return bad;
}

int main() {
    long bad = 0;
    std::vector<uint32_t> ds = {1, 2, 3, 5, 6, 7, 8, 12, 16, 24, 40, 48, 80, 96, 1152, 4608, 9450,
                                27280, 75600, 604800, 65535, 65536, 65537, 1u << 31, 0x7fffffffu,
                                0x80000001u, 0xffffffffu};
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + next32() % 100000);
    for (int i = 0; i < 200; ++i) ds.push_back(1 + next32());
    for (uint32_t d : ds) {
        dtl::FastDiv f = dtl::FastDiv::make(d);
        uint32_t ns[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : ns)
            if (f.div(n) != n / d) { if (bad < 10) printf("fastdiv d=%u n=%u got %u\n", d, n, f.div(n)); ++bad; }
        for (int i = 0; i < 2000; ++i) {
            uint32_t n = next32();
            if (f.div(n) != n / d) { if (bad < 10) printf("fastdiv d=%u n=%u got %u\n", d, n, f.div(n)); ++bad; }
        }
    }
    for (int total = 1; total <= 6000; total += (total < 600 ? 1 : 37)) {
        std::vector<int> seen(total, 0);
        for (int pid = 0; pid < total; ++pid) {
            int l = dtl::xcd_contiguous(pid, total);
            if (l < 0 || l >= total || seen[l]++) { if (bad < 10) printf("xcd total=%d pid=%d -> %d\n", total, pid, l); ++bad; }
        }
    }
    const long Ws[] = {1, 2, 7, 63, 64, 511, 512, 513, 1000, 3888, 41088, 62208, 65537, 2193072};
    const int Gs[] = {1, 2, 3, 7, 64, 216, 511, 512};
    for (long W : Ws)
        for (int G0 : Gs) {
            dtl::StreamK w = {};
            w.G_sk = (int)(W < G0 ? W : G0);
            w.q = W / w.G_sk;
            w.r = (int)(W % w.G_sk);
            if (dtl::sk_first_unit(w, 0) != 0 || dtl::sk_first_unit(w, w.G_sk) != W) { printf("streamk ends W=%ld G=%d\n", W, w.G_sk); ++bad; }
            for (int g = 0; g < w.G_sk; ++g) {
                const long a = dtl::sk_first_unit(w, g), b = dtl::sk_first_unit(w, g + 1);
                if (b - a != w.q + (g < w.r)) { if (bad < 10) printf("streamk size W=%ld G=%d g=%d\n", W, w.G_sk, g); ++bad; }
                const long probes[] = {a, b - 1, (a + b) / 2};
                for (long u : probes)
                    if (dtl::sk_owner(w, u) != g) { if (bad < 10) printf("streamk owner W=%ld G=%d u=%ld\n", W, w.G_sk, u); ++bad; }
            }
        }
    // the schedule: whole tiles first, the split part's ranges partition its units, at most
    // one workgroup per slot, and the workloads land where intended
    const long tiles_l[] = {1, 2, 9, 100, 216, 255, 256, 257, 300, 511, 512, 513, 600, 640, 864, 2955, 5120, 5136, 6000};
    const int nkv_l[] = {1, 7, 8, 9, 16, 18, 63, 64, 65, 72, 148, 427, 1182};
    const long slots_l[] = {4, 8, 64, 512};
    for (long tiles : tiles_l)
        for (int n_kv : nkv_l)
            for (long slots : slots_l) {
                const dtl::StreamK w = dtl::plan_stream_k(tiles, n_kv, slots);
                const long W = (tiles - w.n_dp) * (long)n_kv;
                const bool ok_dp = w.n_dp >= 0 && w.n_dp <= tiles && (W == 0) == (w.G_sk == 0);
                bool ok = ok_dp && w.G_sk <= slots;
                if (w.G_sk > 0)   // a short last round of long tiles
                    ok = ok && w.q >= 1 && dtl::sk_first_unit(w, w.G_sk) == W && w.n_dp % slots == 0 &&
                         n_kv >= 64 && (tiles - w.n_dp) * 4 <= slots;
                if (!ok) { if (bad < 10) printf("plan tiles=%ld n_kv=%d slots=%ld -> n_dp=%d G=%d q=%ld\n", tiles, n_kv, slots, w.n_dp, w.G_sk, w.q); ++bad; }
            }
    {
        const dtl::StreamK ring = dtl::plan_stream_k(216, 18, 512);     // FLUX Ring-4 chunk
        const dtl::StreamK wan = dtl::plan_stream_k(5136, 427, 512);    // Wan2.2-5B
        const dtl::StreamK flux = dtl::plan_stream_k(864, 72, 512);     // FLUX
        const dtl::StreamK cross = dtl::plan_stream_k(5136, 8, 512);    // cross-attention
        if (ring.G_sk != 0 || ring.n_dp != 216) { printf("plan ring\n"); ++bad; }
        if (wan.n_dp != 5120 || wan.G_sk != 512) { printf("plan wan\n"); ++bad; }
        if (flux.G_sk != 0 || flux.n_dp != 864) { printf("plan flux\n"); ++bad; }
        if (cross.G_sk != 0 || cross.n_dp != 5136) { printf("plan cross\n"); ++bad; }
        // forced (DTL_ATTN_SPLIT): 1 splits any remainder of tiles with >= 2 key blocks over
        // at most one workgroup per slot, 0 never splits
        const dtl::StreamK f1 = dtl::plan_stream_k(432, 72, 256, 1);    // FLUX, 8-wave tiles
        const dtl::StreamK f0 = dtl::plan_stream_k(2568, 427, 256, 0);  // Wan2.2-5B, 8-wave tiles
        if (f1.n_dp != 256 || f1.G_sk != 256 || dtl::sk_first_unit(f1, f1.G_sk) != 176L * 72) { printf("plan forced split\n"); ++bad; }
        if (f0.G_sk != 0 || f0.n_dp != 2568) { printf("plan split off\n"); ++bad; }
        for (long tiles : tiles_l)
            for (int n_kv : nkv_l)
                for (long slots : slots_l) {
                    const dtl::StreamK w = dtl::plan_stream_k(tiles, n_kv, slots, 1);
                    const long rem = tiles % slots;
                    const bool want = tiles >= slots && rem > 0 && n_kv >= 2;
                    const long W = (tiles - w.n_dp) * (long)n_kv;
                    const bool ok = want ? (w.n_dp == tiles - rem && w.G_sk == (W < slots ? W : slots) &&
                                            dtl::sk_first_unit(w, w.G_sk) == W)
                                         : (w.n_dp == tiles && w.G_sk == 0);
                    if (!ok) { if (bad < 10) printf("forced plan tiles=%ld n_kv=%d slots=%ld\n", tiles, n_kv, slots); ++bad; }
                }
    }
    // element source of output element o, written out from each map's definition
    auto direct = [](dtl::PermuteKind kind, long p, long B, long N, long H, long D, long o) -> long {
        const long Ns = N / p, Hs = H / p;
        long d = o % D; o /= D;
        long hh = o % Hs; o /= Hs;
        if (kind == dtl::PermuteKind::HeadToSeq) {   // out [s][b][n][j*Hs + hh][d]
            long j = o % p; o /= p;
            long n = o % Ns; o /= Ns;
            long b = o % B; long s = o / B;
            return (((j * B + b) * N + s * Ns + n) * Hs + hh) * D + d;
        }
        long tok = o % N; o /= N;
        long b = o % B; o /= B;
        long s = tok / Ns, n = tok % Ns;
        if (kind == dtl::PermuteKind::SeqToHead) {   // out [j][b][tok][hh][d]
            long j = o;
            return (((s * B + b) * Ns + n) * H + j * Hs + hh) * D + d;
        }
        long c = o % 3; long j = o / 3;              // out [j][c][b][tok][hh][d]
        return ((((s * B + b) * Ns + n) * 3 + c) * H + j * Hs + hh) * D + d;
    };
    const int shapes[][5] = {{1, 1, 3, 2, 4}, {2, 1, 8, 4, 3}, {4, 2, 12, 8, 5}, {4, 1, 16, 24, 2},
                             {3, 1, 9, 6, 7}, {4, 1, 8, 24, 128}, {8, 1, 16, 40, 128}, {2, 3, 6, 2, 64},
                             {5, 2, 10, 5, 8}, {1, 2, 7, 3, 1}, {6, 1, 12, 12, 1}, {2, 1, 4, 4, 6}};
    const dtl::PermuteKind kinds[] = {dtl::PermuteKind::SeqToHead, dtl::PermuteKind::HeadToSeq,
                                      dtl::PermuteKind::QkvSeqToHead};
    const int ebs[] = {1, 2, 4, 8};
    for (auto& sh : shapes)
        for (auto kind : kinds)
            for (int eb : ebs) {
                const int p = sh[0], B = sh[1], N = sh[2], H = sh[3], D = sh[4];
                const dtl::RunMap m = dtl::make_run_map(kind, p, B, N, H, D, eb);
                const long u = dtl::permute_unit_bytes((long)(H / p) * D * eb);
                const long per = u / eb;  // elements per copy unit
                const long elems = dtl::permute_elements(kind, B, N, H, D);
                if ((long)m.total * per != elems) { printf("runmap total\n"); ++bad; continue; }
                std::vector<int> seen(m.total, 0);
                for (uint32_t e = 0; e < m.total; ++e) {
                    const long src = m.source(e);
                    if (src < 0 || src >= (long)m.total || seen[src]++ ||
                        src * per != direct(kind, p, B, N, H, D, (long)e * per)) {
                        if (bad < 10) printf("runmap kind=%d p=%d B=%d N=%d H=%d D=%d eb=%d e=%u src=%ld\n",
                                             (int)kind, p, B, N, H, D, eb, e, src);
                        ++bad;
                    }
                }
            }
    bad += check_tile_layout<128, 4>();
    bad += check_tile_layout<128, 8>();
    bad += check_tile_layout<64, 4>();
    bad += check_tile_layout<64, 8>();
    printf("%s (%ld failures)\n", bad ? "FAIL" : "OK", bad);
    return bad ? 1 : 0;
}
