// C ABI of libdtl.so: host-side validation, then one kernel launch per call.
// Declarations and the contract of each entry point are in include/dtl.h.
#include <math.h>
#include <stdint.h>

#include "dtl.h"
#include "common.h"
#include "runmap.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges)
bool overlap(const void* a, long na, const void* b, long nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

constexpr long kIntMax = 2147483647l;

}  // namespace

extern "C" {

const char* dtl_status_string(dtl_status s) {
    switch (s) {
        case DTL_OK: return "DTL_OK";
        case DTL_ERR_INVALID_ARG: return "DTL_ERR_INVALID_ARG: invalid argument";
        case DTL_ERR_UNSUPPORTED: return "DTL_ERR_UNSUPPORTED: not supported by this build";
        case DTL_ERR_HIP: return "DTL_ERR_HIP: HIP runtime error at launch";
        case DTL_ERR_WORKSPACE:
            return "DTL_ERR_WORKSPACE: the split schedule needs more scratch memory than the "
                   "library's static workspace holds (attn_fwd_lse_noalloc)";
    }
    return "DTL_ERR_UNKNOWN: unknown status";
}

}  // extern "C"

namespace {

// Shared validation and launch of attn_fwd_lse, attn_fwd_lse_accumulate (o_prev set) and
// attn_fwd_lse_kv_chunks (P > 1 chunks: o and lse hold P results).
dtl_status attn_call(const void* q, const void* k, const void* v, const float* o_prev,
                     const float* lse_prev, void* o, float* lse, int B, int Nq, int Nkv, int H,
                     int D, int P, float softmax_scale, dtl_dtype o_dtype, bool accum,
                     hipStream_t stream, bool static_ws = false) {
    if (!q || !k || !v || !o || !lse) return DTL_ERR_INVALID_ARG;
    if (accum && (!o_prev || !lse_prev)) return DTL_ERR_INVALID_ARG;
    if (B <= 0 || Nq <= 0 || Nkv <= 0 || H <= 0 || D <= 0) return DTL_ERR_INVALID_ARG;
    if (P <= 0 || Nkv % P != 0 || (accum && P != 1)) return DTL_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return DTL_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return DTL_ERR_INVALID_ARG;
    if (accum && (!aligned16(o_prev) || !aligned16(lse_prev))) return DTL_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return DTL_ERR_UNSUPPORTED;
    if (o_dtype != DTL_BF16 && o_dtype != DTL_F32) return DTL_ERR_UNSUPPORTED;
    const long q_bytes = (long)B * Nq * H * D * 2;
    const long kv_bytes = (long)B * Nkv * H * D * 2;
    const long o_bytes = (long)P * B * Nq * H * D * (o_dtype == DTL_F32 ? 4 : 2);
    const long l_bytes = (long)P * B * H * Nq * 4;
    if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
        overlap(o, o_bytes, v, kv_bytes) || overlap(o, o_bytes, lse, l_bytes) ||
        overlap(lse, l_bytes, q, q_bytes) || overlap(lse, l_bytes, k, kv_bytes) ||
        overlap(lse, l_bytes, v, kv_bytes))
        return DTL_ERR_INVALID_ARG;
    if (accum) {
        // in place is allowed exactly (o == o_prev with an f32 o, lse == lse_prev); any
        // other overlap of an output with the previous result is rejected
        const long op_bytes = (long)B * Nq * H * D * 4;
        const bool o_same = o == (const void*)o_prev && o_dtype == DTL_F32;
        if ((!o_same && overlap(o, o_bytes, o_prev, op_bytes)) ||
            (lse != lse_prev && overlap(lse, l_bytes, lse_prev, l_bytes)) ||
            overlap(o, o_bytes, lse_prev, l_bytes) || overlap(lse, l_bytes, o_prev, op_bytes))
            return DTL_ERR_INVALID_ARG;
    }
    const long tiles = ((long)Nq + 127) / 128 * H * B * P;
    if (tiles > kIntMax || (long)B * Nkv * H > kIntMax || (long)P * B * Nq * H > kIntMax ||
        (long)H * D > (1l << 24))
        return DTL_ERR_INVALID_ARG;
    // the kernel forms query rows (up to Nq + 254 in a last 256-row tile) and key indices (up
    // to Nkv + 63 for the next key tile) as ints
    if ((long)Nq > kIntMax - 256 || (long)Nkv > kIntMax - 256) return DTL_ERR_INVALID_ARG;
    bool too_small = false;
    hipError_t e = dtl::launch_attn_fwd(q, k, v, o, lse, accum ? o_prev : nullptr,
                                        accum ? lse_prev : nullptr, B, Nq, Nkv, H, D, P,
                                        softmax_scale, o_dtype == DTL_F32, static_ws,
                                        &too_small, stream);
    if (too_small) return DTL_ERR_WORKSPACE;
    return e == hipSuccess ? DTL_OK : DTL_ERR_HIP;
}

}  // namespace

extern "C" {

dtl_status attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Nq, int Nkv, int H, int D, float softmax_scale,
                        dtl_dtype o_dtype, hipStream_t stream) {
    return attn_call(q, k, v, nullptr, nullptr, o, lse, B, Nq, Nkv, H, D, 1, softmax_scale,
                     o_dtype, false, stream);
}

dtl_status attn_fwd_lse_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Nq, int Nkv, int H, int D, float softmax_scale,
                                dtl_dtype o_dtype, hipStream_t stream) {
    return attn_call(q, k, v, nullptr, nullptr, o, lse, B, Nq, Nkv, H, D, 1, softmax_scale,
                     o_dtype, false, stream, true);
}

dtl_status attn_fwd_lse_kv_chunks(const void* q, const void* k, const void* v, void* o_parts,
                                  float* lse_parts, int B, int Nq, int Nkv, int H, int D, int P,
                                  float softmax_scale, dtl_dtype o_dtype, hipStream_t stream) {
    return attn_call(q, k, v, nullptr, nullptr, o_parts, lse_parts, B, Nq, Nkv, H, D, P,
                     softmax_scale, o_dtype, false, stream);
}

dtl_status attn_fwd_lse_accumulate(const void* q, const void* k, const void* v,
                                   const float* o_prev, const float* lse_prev, void* o,
                                   float* lse, int B, int Nq, int Nkv, int H, int D,
                                   float softmax_scale, dtl_dtype o_dtype, hipStream_t stream) {
    return attn_call(q, k, v, o_prev, lse_prev, o, lse, B, Nq, Nkv, H, D, 1, softmax_scale,
                     o_dtype, true, stream);
}

dtl_status attn_merge_lse(const void* o_parts, const float* lse_parts, void* o, float* lse,
                          int P, int B, int N, int H, int D, dtl_dtype parts_dtype,
                          dtl_dtype out_dtype, hipStream_t stream) {
    if (!o_parts || !lse_parts || !o) return DTL_ERR_INVALID_ARG;
    if (P <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0) return DTL_ERR_INVALID_ARG;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || (lse && !aligned16(lse)))
        return DTL_ERR_INVALID_ARG;
    if (D % 8 != 0 || P > dtl::merge_max_parts()) return DTL_ERR_UNSUPPORTED;
    if ((parts_dtype != DTL_BF16 && parts_dtype != DTL_F32) ||
        (out_dtype != DTL_BF16 && out_dtype != DTL_F32))
        return DTL_ERR_UNSUPPORTED;
    const long rows = (long)B * N * H;
    const long parts_bytes = (long)P * rows * D * (parts_dtype == DTL_F32 ? 4 : 2);
    const long lp_bytes = (long)P * rows * 4;
    const long o_bytes = rows * D * (out_dtype == DTL_F32 ? 4 : 2);
    const long l_bytes = rows * 4;
    if (overlap(o, o_bytes, o_parts, parts_bytes) || overlap(o, o_bytes, lse_parts, lp_bytes))
        return DTL_ERR_INVALID_ARG;
    if (lse && (overlap(lse, l_bytes, o_parts, parts_bytes) || overlap(lse, l_bytes, lse_parts, lp_bytes) ||
                overlap(lse, l_bytes, o, o_bytes)))
        return DTL_ERR_INVALID_ARG;
    if (rows * (D / 8) > kIntMax || (long)B * H * N > kIntMax) return DTL_ERR_INVALID_ARG;
    hipError_t e = dtl::launch_merge(o_parts, lse_parts, o, lse, P, B, N, H, D,
                                     parts_dtype == DTL_F32, out_dtype == DTL_F32, stream);
    return e == hipSuccess ? DTL_OK : DTL_ERR_HIP;
}

}  // extern "C"

namespace {

dtl_status permute_call(dtl::PermuteKind kind, const void* in, void* out, int p, int B, int N,
                        int H, int D, int elem_bytes, hipStream_t stream) {
    if (!in || !out) return DTL_ERR_INVALID_ARG;
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0) return DTL_ERR_INVALID_ARG;
    if (N % p != 0 || H % p != 0) return DTL_ERR_INVALID_ARG;
    if (!aligned16(in) || !aligned16(out)) return DTL_ERR_INVALID_ARG;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
        return DTL_ERR_UNSUPPORTED;
    const long elems = dtl::permute_elements(kind, B, N, H, D);
    if (elems > (1l << 40)) return DTL_ERR_INVALID_ARG;  // keeps the byte count below exact
    const long bytes = elems * elem_bytes;
    if (overlap(in, bytes, out, bytes)) return DTL_ERR_INVALID_ARG;
    const int unit = dtl::permute_unit_bytes((long)(H / p) * D * elem_bytes);
    if (bytes / unit > dtl::permute_max_units()) return DTL_ERR_INVALID_ARG;
    hipError_t e = dtl::launch_permute(kind, in, out, p, B, N, H, D, elem_bytes, stream);
    return e == hipSuccess ? DTL_OK : DTL_ERR_HIP;
}

}  // namespace

extern "C" {

dtl_status seq_to_head_permute(const void* in, void* out, int p, int B, int N, int H, int D,
                               int elem_bytes, hipStream_t stream) {
    return permute_call(dtl::PermuteKind::SeqToHead, in, out, p, B, N, H, D, elem_bytes, stream);
}

dtl_status head_to_seq_permute(const void* in, void* out, int p, int B, int N, int H, int D,
                               int elem_bytes, hipStream_t stream) {
    return permute_call(dtl::PermuteKind::HeadToSeq, in, out, p, B, N, H, D, elem_bytes, stream);
}

dtl_status qkv_seq_to_head_permute(const void* in, void* out, int p, int B, int N, int H, int D,
                                   int elem_bytes, hipStream_t stream) {
    return permute_call(dtl::PermuteKind::QkvSeqToHead, in, out, p, B, N, H, D, elem_bytes,
                        stream);
}

dtl_status qkv_norm_rope_permute(const void* qkv, const float* gamma_q, const float* gamma_k,
                                 const float* cos_t, const float* sin_t, void* out, int p, int B,
                                 int N, int H, int D, float eps, hipStream_t stream) {
    if (!qkv || !gamma_q || !gamma_k || !cos_t || !sin_t || !out) return DTL_ERR_INVALID_ARG;
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0) return DTL_ERR_INVALID_ARG;
    if (N % p != 0 || H % p != 0) return DTL_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || !isfinite(eps)) return DTL_ERR_INVALID_ARG;
    if (!aligned16(qkv) || !aligned16(gamma_q) || !aligned16(gamma_k) || !aligned16(cos_t) ||
        !aligned16(sin_t) || !aligned16(out))
        return DTL_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return DTL_ERR_UNSUPPORTED;
    if ((long)H * D > dtl::norm_rope_max_hidden()) return DTL_ERR_UNSUPPORTED;
    if ((long)B * N * 3 > kIntMax / 2) return DTL_ERR_INVALID_ARG;
    const long bytes = (long)B * N * 3 * H * D * 2;
    const long g_bytes = (long)H * D * 4;
    const long t_bytes = (long)N * (D / 2) * 4;
    if (overlap(out, bytes, qkv, bytes) || overlap(out, bytes, gamma_q, g_bytes) ||
        overlap(out, bytes, gamma_k, g_bytes) || overlap(out, bytes, cos_t, t_bytes) ||
        overlap(out, bytes, sin_t, t_bytes))
        return DTL_ERR_INVALID_ARG;
    hipError_t e = dtl::launch_qkv_norm_rope(qkv, gamma_q, gamma_k, cos_t, sin_t, out, p, B, N, H,
                                             D, eps, stream);
    return e == hipSuccess ? DTL_OK : DTL_ERR_HIP;
}

}  // extern "C"
