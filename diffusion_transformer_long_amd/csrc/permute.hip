// Ulysses seq->head permute (gfx950), a bit-exact, bandwidth-bound copy.
//
//   out[j][b][s*(N/p) + n][hh][d] = in[s][b][n][j*(H/p) + hh][d]
//
// the local half of the all-to-all that turns "N/p tokens x all heads" into "all N
// tokens x H/p heads" (arganzheng.life, multi-GPU diffusion parallelism, section 4.1;
// MindIE SD "多卡并行" page, Ulysses usage example).  For fixed (j, b, token) the
// H/p*D elements are contiguous in both tensors, so the copy is a gather of runs.
// Each thread moves 16 B; consecutive threads cover consecutive output bytes, and the
// index math uses multiply-high division by the invariant run and row counts.
#include "common.h"
#include "fastdiv.h"

namespace dtl {
namespace {

constexpr int kThreads = 256;

// 16-byte path: run_vec = (H/p)*D*elem/16 vectors per output row.
__global__ __launch_bounds__(kThreads)
void permute16_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, FastDiv div_run,
                      FastDiv div_n, FastDiv div_ns, FastDiv div_b, uint32_t row_vec_in,
                      uint32_t total_vec) {
    const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= total_vec) return;
    const uint32_t orow = div_run.div(e);          // (j*B + b)*N + tok
    const uint32_t c = e - orow * div_run.d;
    const uint32_t jb = div_n.div(orow);
    const uint32_t tok = orow - jb * div_n.d;
    const uint32_t j = div_b.div(jb);
    const uint32_t b = jb - j * div_b.d;
    const uint32_t s = div_ns.div(tok);
    const uint32_t n = tok - s * div_ns.d;
    // source token row (s, b, n) holds H*D elements = row_vec_in vectors; group j starts at j*run
    const long src = ((long)(s * div_b.d + b) * div_ns.d + n) * row_vec_in + (long)j * div_run.d + c;
    __builtin_nontemporal_store(__builtin_nontemporal_load(in + src), out + e);
}

// Element path for runs that are not a multiple of 16 B.
template <typename E>
__global__ __launch_bounds__(kThreads)
void permute_elem_kernel(const E* __restrict__ in, E* __restrict__ out, int p, int B, long Ns,
                         int H, int Hs, int D, long total) {
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;
    if (e >= total) return;
    const long run = (long)Hs * D;
    const long orow = e / run;
    const long c = e - orow * run;
    const long N = Ns * p;
    const long tok = orow % N;
    const long jb = orow / N;
    const long b = jb % B, j = jb / B;
    const long s = tok / Ns, n = tok % Ns;
    out[e] = in[((s * B + b) * Ns + n) * (long)H * D + j * run + c];
}

}  // namespace

hipError_t launch_permute(const void* in, void* out, int p, int B, int N, int H, int D,
                          int elem_bytes, hipStream_t stream) {
    const long Ns = N / p;
    const int Hs = H / p;
    const long run_bytes = (long)Hs * D * elem_bytes;
    const long total_bytes = (long)N * H * D * elem_bytes * B;
    if (run_bytes % 16 == 0 && total_bytes / 16 < (1l << 31)) {
        const uint32_t run_vec = (uint32_t)(run_bytes / 16);
        const uint32_t total_vec = (uint32_t)(total_bytes / 16);
        const uint32_t row_vec_in = (uint32_t)((long)H * D * elem_bytes / 16);
        const dim3 grid((total_vec + kThreads - 1) / kThreads), block(kThreads);
        permute16_kernel<<<grid, block, 0, stream>>>(
            static_cast<const u32x4*>(in), static_cast<u32x4*>(out), FastDiv::make(run_vec),
            FastDiv::make((uint32_t)N), FastDiv::make((uint32_t)Ns), FastDiv::make((uint32_t)B),
            row_vec_in, total_vec);
        return hipGetLastError();
    }
    const long total = (long)B * N * H * D;
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads)), block(kThreads);
    switch (elem_bytes) {
        case 1: permute_elem_kernel<uint8_t><<<grid, block, 0, stream>>>(static_cast<const uint8_t*>(in), static_cast<uint8_t*>(out), p, B, Ns, H, Hs, D, total); break;
        case 2: permute_elem_kernel<uint16_t><<<grid, block, 0, stream>>>(static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), p, B, Ns, H, Hs, D, total); break;
        case 4: permute_elem_kernel<uint32_t><<<grid, block, 0, stream>>>(static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out), p, B, Ns, H, Hs, D, total); break;
        default: permute_elem_kernel<uint64_t><<<grid, block, 0, stream>>>(static_cast<const uint64_t*>(in), static_cast<uint64_t*>(out), p, B, Ns, H, Hs, D, total); break;
    }
    return hipGetLastError();
}

}  // namespace dtl
