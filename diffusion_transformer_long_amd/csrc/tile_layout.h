// LDS layout of the attention kernel's key tiles (64 keys of K and of V, bf16, head_dim 64
// or 128): where the direct global -> LDS loads put each 16-byte piece, and the fragment
// reads that feed v_mfma_f32_32x32x16_bf16.  The kernel takes every offset from here; the
// host check (tests/host) proves that the reads return the operand elements the MFMAs
// need, that the loads fill each tile exactly once, and that every read is free of LDS
// bank conflicts (64 banks of 4 bytes).
#pragma once

#include "common.h"

namespace dtl {

// LDS row m of a K tile holds key krow_slot(m) of the tile: bits 2 and 3 swapped (an
// involution).  With this order the S^T = K Q^T accumulator of lane l holds, in register
// i, key 16*(i/8) + 8*(l/32) + i%8 of its 32-key half, which is the B-operand order of
// the P.V product, so P goes from the S registers to the MFMA without a shuffle.
__host__ __device__ constexpr int krow_slot(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// NW: waves of the workgroup that loads the tile (4 or 8); each fills 64 / NW rows.
template <int D, int NW>
struct TileLayout {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static constexpr int kKeys = 64;            // keys per tile
    static constexpr int kRowBytes = 2 * D;     // one key's row
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;   // rows one 1 KB load instruction fills
    static constexpr int kRowsPerWave = kKeys / NW;
    static constexpr int kLoadsPerWave = kRowsPerWave / kRowsPerLoad;   // per tensor
    static_assert(kLoadsPerWave >= 1, "a wave fills whole load blocks");
    static constexpr int kTileBytes = kKeys * kRowBytes;

    // XOR swizzles of the 16-byte chunk index within a row: chunk c of K row m sits at
    // position c ^ fk(m), chunk c of V row m at c ^ 4 fv(m).
    __host__ __device__ static constexpr int fk(int m) { return D == 128 ? (m & 15) : ((m >> 1) & 7); }
    __host__ __device__ static constexpr int fv(int m) { return D == 128 ? (m & 3) : ((m >> 1) & 1); }

    // Load instruction i of wave w writes the 1 KB block starting at load_block(w, i); its
    // lane l writes bytes [16 l, 16 l + 16) of it: row load_row(w, i, l), position l % kChunks.
    __host__ __device__ static constexpr int load_block(int w, int i) {
        return (kRowsPerWave * w + kRowsPerLoad * i) * kRowBytes;
    }
    __host__ __device__ static constexpr int load_row(int w, int i, int l) {
        return kRowsPerWave * w + kRowsPerLoad * i + l / kChunks;
    }
    // What that lane loads: the key (within the tile) and the 16-byte chunk of its row.
    __host__ __device__ static constexpr int k_src_key(int w, int i, int l) { return krow_slot(load_row(w, i, l)); }
    __host__ __device__ static constexpr int k_src_chunk(int w, int i, int l) {
        return (l % kChunks) ^ fk(load_row(w, i, l));
    }
    __host__ __device__ static constexpr int v_src_key(int w, int i, int l) { return load_row(w, i, l); }
    __host__ __device__ static constexpr int v_src_chunk(int w, int i, int l) {
        return (l % kChunks) ^ (4 * fv(load_row(w, i, l)));
    }

    // K fragment (A operand of S^T = K Q^T) for key half kb and k-step ks: lane l reads row
    // kb*32 + l%32, chunk 2 ks + l/32 (head_dim 16 ks + 8 (l/32) .. +7), one 16-byte read.
    // The swizzle only touches chunk bits, so the offset is k_lane(l) ^ 32 ks.
    __host__ __device__ static constexpr int k_lane(int l) {
        const int r = l & 31, g = l >> 5, f = fk(r);
        return r * kRowBytes + 32 * (f >> 1) + 16 * (g ^ (f & 1));
    }
    __host__ __device__ static constexpr int k_frag(int kb, int ks, int l) {
        return kb * 32 * kRowBytes + (k_lane(l) ^ (ks << 5));
    }

    // V^T fragment (A operand of O^T += V^T P^T) for key half kb, 16-key group hf and
    // head_dim block db: lane l needs keys kb*32 + hf*16 + 8 (l/32) .. +7 of column
    // db*32 + l%32.  Two transposing 8-byte reads (j = 0, 1) give 4 keys each: in each
    // group of 16 lanes, lane l addresses key kb*32 + hf*16 + 8 (l/32) + 4 j + (l%16)/4,
    // columns db*32 + 16 ((l/16)%2) + 4 (l%4) .. +3, and receives column l%16 of the
    // group's 4 x 16 block.  The swizzle again only touches chunk bits: v_lane(l) ^ 64 db.
    __host__ __device__ static constexpr int v_lane(int l) {
        const int qv = (l & 15) >> 2;
        return (8 * (l >> 5) + qv) * kRowBytes + 64 * fv(qv) + 32 * ((l >> 4) & 1) + 16 * ((l >> 1) & 1) +
               8 * (l & 1);
    }
    __host__ __device__ static constexpr int v_frag(int kb, int hf, int db, int j, int l) {
        return (kb * 32 + hf * 16 + 4 * j) * kRowBytes + (v_lane(l) ^ (db << 6));
    }
};

}  // namespace dtl
