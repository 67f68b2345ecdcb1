// Index maps of the Ulysses permutes as copies of contiguous runs.
//
// With Ns = N/p and Hs = H/p, each of the three maps moves runs of Hs*D elements (one
// head group of one token), contiguous in source and destination alike:
//   seq->head   out[j][b][s*Ns + n][hh][:]    = in[s][b][n][j*Hs + hh][:]
//   head->seq   out[s][b][n][j*Hs + hh][:]    = in[j][b][s*Ns + n][hh][:]
//   fused QKV   out[j][c][b][s*Ns + n][hh][:] = in[s][b][n][c][j*Hs + hh][:]
// (arganzheng.life, multi-GPU diffusion parallelism, section 4.1 and its figure: one
// all-to-all before attention and one for O after it; MindIE SD "多卡并行" page, Ulysses
// usage example: split heads / exchange / concatenate tokens, then split tokens /
// exchange / concatenate heads; "AIGC 分布式推理：从 Wan2.2 理解 DP/TP/CP/SP/PP", CP
// section: Q, K and V go in one fused all-to-all).
//
// The output is the runs back to back.  A RunMap gives the source of output run r as
// sum_k digit_k(r) * stride_k over the mixed-radix digits of r (innermost first; the
// quotient left after four digits is digit 4).  Offsets count copy units: the largest of
// 16, 8, 4, 2, 1 bytes dividing the run, so every run start is unit-aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace dtl {

struct RunMap {
    FastDiv run;          // units per run
    FastDiv radix[4];     // digits 0..3 of the output run index, innermost first
    uint32_t stride[5];   // source units per step of digit k (k = 4: the quotient)
    uint32_t total;       // units in the output (and in the input)

    // Source unit of output unit e < total.
    __host__ __device__ __forceinline__ long source(uint32_t e) const {
        uint32_t r = run.div(e);
        long src = (long)(e - r * run.d);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q = radix[k].div(r);
            src += (long)(r - q * radix[k].d) * stride[k];
            r = q;
        }
        return src + (long)r * stride[4];
    }
};

enum class PermuteKind { SeqToHead, HeadToSeq, QkvSeqToHead };

// Copy unit (bytes) of a permute with runs of `run_bytes`.
__host__ inline int permute_unit_bytes(long run_bytes) {
    int u = 16;
    while (run_bytes % u != 0) u >>= 1;
    return u;
}

// Elements moved by one permute call (the input size, equal to the output size).
__host__ inline long permute_elements(PermuteKind kind, int B, int N, int H, int D) {
    return (long)B * N * H * D * (kind == PermuteKind::QkvSeqToHead ? 3 : 1);
}

// The map of `kind` for sizes that the caller has validated (p | N, p | H) and whose
// unit count fits in 32 bits.
__host__ inline RunMap make_run_map(PermuteKind kind, int p, int B, int N, int H, int D,
                                    int elem_bytes) {
    const long Ns = N / p, Hs = H / p;
    const long run_b = Hs * D * elem_bytes;
    const int u = permute_unit_bytes(run_b);
    const uint32_t run = (uint32_t)(run_b / u);
    const uint32_t row = (uint32_t)((long)H * D * elem_bytes / u);  // one token, all heads
    uint32_t rad[4], str[5];
    switch (kind) {
        case PermuteKind::SeqToHead:  // output runs (j, b, s, n), source [s][b][n][j]
            rad[0] = Ns; str[0] = row;
            rad[1] = p;  str[1] = (uint32_t)(B * Ns) * row;
            rad[2] = B;  str[2] = (uint32_t)Ns * row;
            rad[3] = p;  str[3] = run;
            str[4] = 0;
            break;
        case PermuteKind::HeadToSeq:  // output runs (s, b, n, j), source [j][b][s*Ns + n]
            rad[0] = p;  str[0] = (uint32_t)((long)B * N) * run;
            rad[1] = Ns; str[1] = run;
            rad[2] = B;  str[2] = (uint32_t)N * run;
            rad[3] = p;  str[3] = (uint32_t)Ns * run;
            str[4] = 0;
            break;
        case PermuteKind::QkvSeqToHead:  // output runs (j, c, b, s, n), source [s][b][n][c][j]
        default:
            rad[0] = Ns; str[0] = 3 * row;
            rad[1] = p;  str[1] = (uint32_t)(B * Ns) * 3 * row;
            rad[2] = B;  str[2] = (uint32_t)Ns * 3 * row;
            rad[3] = 3;  str[3] = row;
            str[4] = run;
            break;
    }
    RunMap m;
    m.run = FastDiv::make(run);
    for (int k = 0; k < 4; ++k) m.radix[k] = FastDiv::make(rad[k]);
    for (int k = 0; k < 5; ++k) m.stride[k] = str[k];
    m.total = (uint32_t)(permute_elements(kind, B, N, H, D) * elem_bytes / u);
    return m;
}

}  // namespace dtl
