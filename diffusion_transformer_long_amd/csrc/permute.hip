// Ulysses permutes (gfx950): bit-exact, bandwidth-bound copies of contiguous runs.
//
// The three maps (sequence shards -> head shards before attention, head shards ->
// sequence shards for O after it, and Q, K, V together in one pass) and the RunMap that
// describes each are in runmap.h.  One kernel serves all of them: each thread moves one
// copy unit, or four for small copies (16 B whenever a run is a multiple of 16 B); consecutive threads write
// consecutive output units and read whole runs, so loads and stores are both coalesced;
// the index math is multiply-high division by the invariant radices.  Loads and stores
// are nontemporal: every byte is touched once.
#include "common.h"
#include "runmap.h"

namespace dtl {
namespace {

constexpr int kThreads = 256;

// Copies up to this many bytes are bound by memory latency and ramp-up rather than by
// HBM bandwidth: there each thread moves UPT = 4 units, all four loads in flight before
// the stores (FLUX Ulysses-4, 56.6 MB: 11.3 against 11.9 us); larger ones keep one unit
// per thread (Wan2.1-14B Ulysses-8, 1.55 GB: 247 against 252 us with four).
constexpr long kSmallCopyBytes = 256l << 20;

// Thread i of workgroup b moves output units b * UPT * kThreads + j * kThreads + i,
// j < UPT (consecutive threads on consecutive units for every j).
template <typename U, int UPT>
__global__ __launch_bounds__(kThreads)
void run_copy_kernel(const U* __restrict__ in, U* __restrict__ out, RunMap m) {
    const uint32_t e0 = blockIdx.x * (UPT * kThreads) + threadIdx.x;
    U x[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const uint32_t e = e0 + j * kThreads;
        if (e < m.total) x[j] = __builtin_nontemporal_load(in + m.source(e));
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const uint32_t e = e0 + j * kThreads;
        if (e < m.total) __builtin_nontemporal_store(x[j], out + e);
    }
}

template <typename U>
hipError_t launch_run_copy(const void* in, void* out, const RunMap& m, hipStream_t stream) {
    const bool small = (long)m.total * (long)sizeof(U) <= kSmallCopyBytes;
    const int upt = small ? 4 : 1;
    const dim3 grid((uint32_t)(((long)m.total + upt * kThreads - 1) / (upt * kThreads))), block(kThreads);
    if (small)
        run_copy_kernel<U, 4><<<grid, block, 0, stream>>>(static_cast<const U*>(in), static_cast<U*>(out), m);
    else
        run_copy_kernel<U, 1><<<grid, block, 0, stream>>>(static_cast<const U*>(in), static_cast<U*>(out), m);
    return hipGetLastError();
}

}  // namespace

long permute_max_units() { return (1l << 31) - kThreads; }

hipError_t launch_permute(PermuteKind kind, const void* in, void* out, int p, int B, int N,
                          int H, int D, int elem_bytes, hipStream_t stream) {
    const RunMap m = make_run_map(kind, p, B, N, H, D, elem_bytes);
    switch (permute_unit_bytes((long)(H / p) * D * elem_bytes)) {
        case 16: return launch_run_copy<u32x4>(in, out, m, stream);
        case 8: return launch_run_copy<u32x2>(in, out, m, stream);
        case 4: return launch_run_copy<uint32_t>(in, out, m, stream);
        case 2: return launch_run_copy<uint16_t>(in, out, m, stream);
        default: return launch_run_copy<uint8_t>(in, out, m, stream);
    }
}

}  // namespace dtl
