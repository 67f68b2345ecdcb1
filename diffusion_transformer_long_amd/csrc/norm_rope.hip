// QK-RMSNorm + rotary position embedding, fused with the Ulysses fused-QKV permute
// (gfx950), one HBM pass: bandwidth-bound.
//
// For token t = s*(N/p) + n of sequence shard s and c = q or k, over the token's H*D
// hidden values x (the norm spans all heads: "AIGC 分布式推理：从 Wan2.2 理解
// DP/TP/CP/SP/PP", TP section; RoPE acts by token position and the cos/sin tables are
// sliced with the tokens: same page, TP and CP sections):
//     y_e = x_e * gamma_c[e] / sqrt(mean(x^2) + eps)
//     per head and pair i: (y_2i, y_2i+1) -> (y_2i cos[t][i] - y_2i+1 sin[t][i],
//                                          y_2i sin[t][i] + y_2i+1 cos[t][i])
// v is copied.  Rows are read from the fused QKV projection's layout [p,B,N/p,3,H,D] and
// written to the head shards [p,3,B,N,H/p,D] that attention takes (out[j][c] is head
// group j's q, k or v), so the norm, the rotation and the all-to-all's local data
// movement cost one read and one write of Q, K and V.
//
// One wave per (token, tensor): the wave holds the token's H*D values as 16-byte chunks
// (8 bf16; chunk ci = lane + 64*k), reduces the sum of squares across the wave, then
// scales, rotates (pairs never straddle a chunk) and stores each chunk to its head's
// destination row.  Arithmetic in f32, rounded to bf16 to nearest even once.
#include "common.h"
#include "fastdiv.h"

namespace dtl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxChunksPerLane = 16;   // H*D <= 8192
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the wave: DPP within each row of 16 lanes (xor 1, xor 2, then the half-row and
// row mirrors), then the four row sums read as scalars.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror
    x += dpp<0x140>(x);   // row_mirror
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
}

// CPL: chunks per lane the wave holds (H*D <= 512*CPL), a template parameter so that the
// registers follow the row length.  At least 4 waves per SIMD keep enough loads in flight
// (2 for the longest rows, which would spill at 4).
template <int D, int CPL>
__global__ __launch_bounds__(kThreads, CPL <= 10 ? 4 : 2)
void qkv_norm_rope_kernel(const u32x4* __restrict__ in, const float* __restrict__ gamma_q,
                          const float* __restrict__ gamma_k, const float* __restrict__ cs,
                          const float* __restrict__ sn, u32x4* __restrict__ out, int B, int N,
                          int H, FastDiv div_ns, FastDiv div_hs, int items, float eps) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * kWaves + wave;   // = source row (token-major, then c)
    if (item >= items) return;
    const int tok = item / 3;                      // (s*B + b)*Ns + n
    const int c = item - 3 * tok;
    const uint32_t Ns = div_ns.d;
    const uint32_t sb = div_ns.div((uint32_t)tok);
    const uint32_t n = (uint32_t)tok - sb * Ns;
    const uint32_t s = sb / (uint32_t)B;
    const uint32_t b = sb - s * (uint32_t)B;
    const uint32_t t = s * Ns + n;                 // position in the whole sequence
    const int HD = H * D;
    const int nch = HD / 8;
    const uint32_t Hs = div_hs.d;
    const u32x4* src = in + (long)item * nch;

    // destination chunk of source chunk ci (head h = ci / (D/8), group j = h / Hs)
    auto dst_of = [&](int ci) -> long {
        const uint32_t h = (uint32_t)ci / (D / 8);
        const uint32_t j = div_hs.div(h);
        const uint32_t hh = h - j * Hs;
        const long row = (((long)(j * 3 + c) * B + b) * N + t) * Hs + hh;
        return row * (D / 8) + (ci - (int)h * (D / 8));
    };

    u32x4 x[CPL];   // all of the row's loads are issued before the first use
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int ci = lane + 64 * k;
        if (ci < nch) x[k] = __builtin_nontemporal_load(src + ci);
    }
    if (c == 2) {   // v: the permute alone
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int ci = lane + 64 * k;
            if (ci < nch) __builtin_nontemporal_store(x[k], out + dst_of(ci));
        }
        return;
    }

    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int ci = lane + 64 * k;
        if (ci < nch) {
            const f32x8 v = __builtin_convertvector(__builtin_bit_cast(bf16x8, x[k]), f32x8);
            ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3] +
                  v[4] * v[4] + v[5] * v[5] + v[6] * v[6] + v[7] * v[7];
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)HD + eps);
    const float* gamma = c == 0 ? gamma_q : gamma_k;
    // every chunk of a lane sits at the same place within its head (64 lanes x 8 elements
    // are whole heads), so the lane's cos/sin values are the same for all its chunks
    static_assert(512 % D == 0, "a wave's 512 elements are whole heads");
    const int i0 = ((lane * 8) % D) / 2;           // first pair of the lane's chunks within a head
    const f32x4 co = *reinterpret_cast<const f32x4*>(cs + (long)t * (D / 2) + i0);
    const f32x4 si = *reinterpret_cast<const f32x4*>(sn + (long)t * (D / 2) + i0);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int ci = lane + 64 * k;
        if (ci < nch) {
            const int e0 = ci * 8;                 // first element (h*D + d0)
            const f32x8 v = __builtin_convertvector(__builtin_bit_cast(bf16x8, x[k]), f32x8);
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + e0);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + e0 + 4);
            const float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            f32x8 y;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = v[2 * q] * r * gg[2 * q];
                const float bb = v[2 * q + 1] * r * gg[2 * q + 1];
                y[2 * q] = a * co[q] - bb * si[q];
                y[2 * q + 1] = a * si[q] + bb * co[q];
            }
            const bf16x8 o = __builtin_convertvector(y, bf16x8);
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), out + dst_of(ci));
        }
    }
}

template <int D, int CPL>
void launch_cpl(const u32x4* in, const float* gq, const float* gk, const float* cs,
                const float* sn, u32x4* o, int B, int N, int H, FastDiv dns, FastDiv dhs,
                int items, float eps, hipStream_t stream) {
    const dim3 grid((items + kWaves - 1) / kWaves), block(kThreads);
    qkv_norm_rope_kernel<D, CPL><<<grid, block, 0, stream>>>(in, gq, gk, cs, sn, o, B, N, H, dns,
                                                            dhs, items, eps);
}

template <int D>
void launch_d(const u32x4* in, const float* gq, const float* gk, const float* cs,
              const float* sn, u32x4* o, int B, int N, int H, FastDiv dns, FastDiv dhs,
              int items, float eps, hipStream_t stream) {
    const int cpl = (H * D / 8 + 63) / 64;
    if (cpl <= 2) launch_cpl<D, 2>(in, gq, gk, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    else if (cpl <= 4) launch_cpl<D, 4>(in, gq, gk, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    else if (cpl <= 8) launch_cpl<D, 8>(in, gq, gk, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    else if (cpl <= 10) launch_cpl<D, 10>(in, gq, gk, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    else launch_cpl<D, kMaxChunksPerLane>(in, gq, gk, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
}

}  // namespace

int norm_rope_max_hidden() { return kMaxChunksPerLane * 64 * 8; }

hipError_t launch_qkv_norm_rope(const void* qkv, const float* gamma_q, const float* gamma_k,
                                const float* cs, const float* sn, void* out, int p, int B,
                                int N, int H, int D, float eps, hipStream_t stream) {
    const int Ns = N / p;
    const int items = p * B * Ns * 3;   // the caller has checked that this fits an int
    const FastDiv dns = FastDiv::make((uint32_t)Ns), dhs = FastDiv::make((uint32_t)(H / p));
    auto in = static_cast<const u32x4*>(qkv);
    auto o = static_cast<u32x4*>(out);
    if (D == 128)
        launch_d<128>(in, gamma_q, gamma_k, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    else
        launch_d<64>(in, gamma_q, gamma_k, cs, sn, o, B, N, H, dns, dhs, items, eps, stream);
    return hipGetLastError();
}

}  // namespace dtl
