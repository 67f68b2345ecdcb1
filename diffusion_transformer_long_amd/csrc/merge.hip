// LSE merge of P partial attention results (gfx950), bandwidth-bound.
//
// For each (b, n, h): L = ln sum_t exp(lse_t), o = sum_t exp(lse_t - L) o_t — the
// online-softmax accumulation of Ring attention across its rounds (arganzheng.life,
// multi-GPU diffusion parallelism, section 4.2; MindIE SD "多卡并行" page, Ring
// Sequence Parallel section).
//
// One thread owns 8 consecutive head_dim values of one row and streams them from
// all P parts (32 B per part in f32), so a wave reads whole 1 KB segments per part.
// Row weights are computed per thread from the P lse values, which every thread of
// the row loads from the same addresses (one cache line, broadcast).
#include "common.h"
#include "fastdiv.h"

namespace dtl {
namespace {

constexpr int kThreads = 256;
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_ __attribute__((ext_vector_type(8)));

template <bool PARTS_F32>
__device__ __forceinline__ f32x8 load8(const void* base, long off) {
    if constexpr (PARTS_F32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
        f32x4 a = __builtin_nontemporal_load(p);
        f32x4 b = __builtin_nontemporal_load(p + 1);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
        u32x4 a = __builtin_nontemporal_load(p);
        return __builtin_convertvector(__builtin_bit_cast(bf16x8_, a), f32x8);
    }
}

template <bool PARTS_F32, bool OUT_F32>
__global__ __launch_bounds__(kThreads)
void merge_kernel(const void* __restrict__ o_parts, const float* __restrict__ lse_parts,
                  void* __restrict__ o, float* __restrict__ lse, int P, FastDiv div_vpr,
                  FastDiv div_h, FastDiv div_n, uint32_t total_vec, long part_o, long part_l, int D) {
    const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= total_vec) return;
    const uint32_t row = div_vpr.div(e);          // (b*N + n)*H + h
    const uint32_t c = e - row * div_vpr.d;       // which 8-value group of the row
    const uint32_t bn = div_h.div(row);
    const uint32_t hh = row - bn * div_h.d;
    const uint32_t b = div_n.div(bn);
    const uint32_t n = bn - b * div_n.d;
    const long li = ((long)b * div_h.d + hh) * div_n.d + n;   // [B, H, N] index
    const long off = (long)row * D + c * 8;

    float M = -INFINITY;
    for (int t = 0; t < P; ++t) M = fmaxf(M, lse_parts[t * part_l + li]);

    f32x8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (M != -INFINITY) {
        float sum = 0.f;
        for (int t = 0; t < P; ++t) sum += __expf(lse_parts[t * part_l + li] - M);
        L = M + __logf(sum);
        for (int t = 0; t < P; ++t) {
            const float lt = lse_parts[t * part_l + li];
            if (lt == -INFINITY) continue;   // an empty part adds nothing
            const float w = __expf(lt - L);
            acc += w * load8<PARTS_F32>(o_parts, t * part_o + off);
        }
    }
    if constexpr (OUT_F32) {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(o) + off);
        __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, p);
        __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, p + 1);
    } else {
        bf16x8_ x = __builtin_convertvector(acc, bf16x8_);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x),
                                    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o) + off));
    }
    if (lse != nullptr && c == 0) lse[li] = L;
}

}  // namespace

hipError_t launch_merge(const void* o_parts, const float* lse_parts, void* o, float* lse,
                        int P, int B, int N, int H, int D, bool parts_f32, bool out_f32,
                        hipStream_t stream) {
    const long rows = (long)B * N * H;
    const uint32_t vpr = (uint32_t)(D / 8);
    const uint32_t total_vec = (uint32_t)(rows * vpr);  // the caller has checked < 2^31
    const long part_o = rows * D;
    const long part_l = rows;
    const FastDiv dv = FastDiv::make(vpr), dh = FastDiv::make((uint32_t)H), dn = FastDiv::make((uint32_t)N);
    const dim3 grid((total_vec + kThreads - 1) / kThreads), block(kThreads);
    if (parts_f32) {
        if (out_f32)
            merge_kernel<true, true><<<grid, block, 0, stream>>>(o_parts, lse_parts, o, lse, P, dv, dh, dn, total_vec, part_o, part_l, D);
        else
            merge_kernel<true, false><<<grid, block, 0, stream>>>(o_parts, lse_parts, o, lse, P, dv, dh, dn, total_vec, part_o, part_l, D);
    } else {
        if (out_f32)
            merge_kernel<false, true><<<grid, block, 0, stream>>>(o_parts, lse_parts, o, lse, P, dv, dh, dn, total_vec, part_o, part_l, D);
        else
            merge_kernel<false, false><<<grid, block, 0, stream>>>(o_parts, lse_parts, o, lse, P, dv, dh, dn, total_vec, part_o, part_l, D);
    }
    return hipGetLastError();
}

}  // namespace dtl
