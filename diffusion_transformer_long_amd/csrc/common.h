// Internal declarations shared by the HIP sources of libdtl.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// gfx950 dispatches consecutive workgroup ids round-robin over its 8 XCDs, each with
// its own L2.  Remapping the id so that each XCD receives one contiguous range of
// logical tiles keeps the tiles that share K/V (same head) on the same L2.
constexpr int kNumXcd = 8;

__host__ __device__ __forceinline__ int xcd_contiguous(int pid, int total) {
    const int per = (total + kNumXcd - 1) / kNumXcd;
    const int rem = total % kNumXcd;
    const int full = rem == 0 ? kNumXcd : rem;  // XCDs that receive `per` ids
    const int xcd = pid % kNumXcd;
    const int local = pid / kNumXcd;
    if (xcd < full) return xcd * per + local;
    return full * per + (xcd - full) * (per - 1) + local;
}

// Launchers (validated arguments only; each returns hipGetLastError()).
// o_prev == nullptr: a fresh result; otherwise continue from (o_prev, lse_prev).  P > 1
// (fresh results only): the keys are P equal chunks, o and lse hold one result per
// (chunk, batch), chunk-major.  static_ws: a split schedule's workspace is the library's
// static device array instead of the pool (nothing is allocated); when the schedule
// needs more than that array holds, nothing is launched, *ws_too_small is set and
// hipErrorInvalidValue returned.
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           const float* o_prev, const float* lse_prev, int B, int Nq, int Nkv,
                           int H, int D, int P, float scale, bool out_f32, bool static_ws,
                           bool* ws_too_small, hipStream_t stream);
int merge_max_parts();  // largest P attn_merge_lse accepts
hipError_t launch_merge(const void* o_parts, const float* lse_parts, void* o, float* lse,
                        int P, int B, int N, int H, int D, bool parts_f32, bool out_f32,
                        hipStream_t stream);
int norm_rope_max_hidden();  // largest H*D qkv_norm_rope_permute accepts
hipError_t launch_qkv_norm_rope(const void* qkv, const float* gamma_q, const float* gamma_k,
                                const float* cs, const float* sn, void* out, int p, int B,
                                int N, int H, int D, float eps, hipStream_t stream);
enum class PermuteKind;
long permute_max_units();  // largest copy-unit count one permute call may move
hipError_t launch_permute(PermuteKind kind, const void* in, void* out, int p, int B, int N,
                          int H, int D, int elem_bytes, hipStream_t stream);

}  // namespace dtl
