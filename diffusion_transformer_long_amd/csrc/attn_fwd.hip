// Attention forward with per-row log-sum-exp for gfx950 (MI355X).
//
// Computes o = softmax(q k^T * scale) v and lse = ln sum_j exp(scale q.k_j) per
// (batch, head, query row), non-causal, on BSND bf16 tensors (MindIE SD "多卡并行"
// page, Ring Sequence Parallel usage example, for the formula; "AIGC 分布式推理：从
// Wan2.2 理解 DP/TP/CP/SP/PP", CP section, for head independence and every query
// seeing every key).  The key loop is the online-softmax accumulation that Ring
// attention also performs across rounds (arganzheng.life, multi-GPU diffusion
// parallelism, section 4.2).
//
// Work decomposition
//   workgroup = NW waves (4 or 8) = 32 NW query rows of one (batch, head); wave w owns
//   rows [32w, 32w+32).  Keys are consumed 64 per iteration from a double-buffered LDS tile.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] B[16x32]):
//   S^T = K Q^T:  A = a 32-key block of K (lane l: key row l%32, 8 head_dim values
//                 at 8*(l/32)), B = Q^T (lane l: query l%32, the same 8 head_dim).
//                 The result puts one query per lane: lane l holds 16 keys of query
//                 l%32, the other 16 keys of that query sit in lane l^32.  Row max and
//                 row sum are in-lane plus one exchange between the lane halves.
//   O^T += V^T P^T: B = P^T comes straight from the S^T registers (rounded to bf16),
//                 because the B operand layout (lane l: column l%32, 8 consecutive k)
//                 matches them once K rows are stored in LDS in a permuted order (rows
//                 m and sigma(m) swap bits 2 and 3), so that register i of lane l holds
//                 key 16*(i/8) + 8*(l/32) + i%8 of its 32-key block.  A = V^T needs 8
//                 consecutive keys of one head_dim column per lane: V stays key-major in
//                 LDS and two transposing reads (ds_read_b64_tr_b16) build it.
//   The O^T accumulator also keeps one query per lane, so the softmax rescale is a
//   per-lane scalar.
//
// Softmax in base 2: p = exp2(s * scale*log2(e) - m), m a reference max of the scaled
// logits in log2 units.  A 32-key half's weights are first taken against the current
// reference; only when some lane's sum of its 16 weights exceeds 2^kRescaleThreshold (or is
// +inf or NaN, as in a row's first half) is the reference moved to a little above the half's
// row max, the accumulators rescaled and the weights taken again.  So p <= 2^threshold always, which
// f32 and bf16 hold without overflow, and the row max is formed only on that rare path.  The row sum is taken over the bf16-rounded weights (two per v_dot2 against
// (1, 1)), i.e. over exactly the weights the P.V product uses.  The result is the same
// softmax, since numerator and denominator share the reference m.
//
// Each key tile runs as four blocks that pair MFMAs with VALU work independent of them
// (S of key half 0; S of half 1 with the softmax of half 0; P.V of half 0 with the
// softmax of half 1; P.V of half 1), since a wave issues in order and VALU work only
// overlaps an MFMA when it sits between MFMAs in the instruction stream.  The loads of
// the next tile are issued after the first block.
//
// K and V tiles go from global memory straight into LDS (global_load_lds_dwordx4: each
// lane of an instruction fills 16 bytes of a 1 KB block; its source address picks the
// piece), so staging takes no registers and no VALU work.  The layout (XOR-swizzled 16-byte
// chunks, conflict-free reads) is in tile_layout.h.  Full tiles load without bounds checks
// from a uniform tile base plus per-lane offsets fixed for the whole loop; the ragged last
// tile repeats its last key for rows past the end (finite values whose logits are masked).
#include <atomic>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "streamk.h"
#include "tile_layout.h"

namespace dtl {
namespace {

// A workgroup has NW waves of 32 query rows (a 32 NW-row query tile): NW = 4, two
// workgroups per CU, in general; NW = 8, one per CU, where the key range is long and the
// 256-row tiles still fill the GPU, since every K/V tile then feeds twice the query rows
// (measured 5.5% faster at FLUX N=4608, 1.6% at Wan2.2-5B, 2% at the Wan2.1-14B chunk, but
// slower at 512 keys and at 1152 x 1152 Ring chunks, which keep NW = 4).
constexpr int kBlockN = 64;            // keys per iteration
// Weights are kept at most 2^this: the running max moves only when a tile half's weights
// against it would exceed that (log2 units; tested on each lane's sum of its weights).
// A larger threshold skips more accumulator rescales; the dominant weight of a peaked row
// is then exp2(x) with x in (0, threshold] instead of exactly 1, whose bf16 rounding the
// rounded-weight row sum below cancels (with an f32 row sum a threshold of 8 would triple
// the worst-case error at FLUX-like logits, std 3).  Weights stay below 2^8, well inside
// the range of bf16 and of the f32 accumulators.
#ifndef DTL_RESCALE_THRESHOLD
#define DTL_RESCALE_THRESHOLD 8.0f
#endif
constexpr float kRescaleThreshold = DTL_RESCALE_THRESHOLD;
static_assert(kRescaleThreshold == (float)(int)kRescaleThreshold && kRescaleThreshold >= 0.0f,
              "a whole number of doublings");
constexpr float pow2_int(int n) { return n == 0 ? 1.0f : 2.0f * pow2_int(n - 1); }
// the same bound on a lane's sum of 16 weights (2^kRescaleThreshold)
constexpr float kMaxLaneSum = pow2_int((int)kRescaleThreshold);
// When the reference moves, it goes this far (log2 units) above the half's row max: the
// weights are floating point, so scaling them all by 2^-4 costs no precision, and later
// keys must then exceed that max by more (about 8 to 12 units instead of 4 to 8) before the
// reference moves again (peaked FLUX-like rows: 6% faster on 1152-key Ring chunks).
constexpr float kHeadroom = 4.0f;
// A tile's finaliser polls its helpers' flags at most this often (s_sleep 8 between
// polls, ~0.2 us; the bound is ~4 ms), then computes the missing keys itself.  The host
// may lower the bound (DTL_ATTN_MAX_POLLS), which changes only who computes those keys.
constexpr int kMaxPolls = 20000;

typedef float f32x8 __attribute__((ext_vector_type(8)));

// max over the two lane halves (lanes l and l^32 hold the two halves of one query row)
__device__ __forceinline__ float halves_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

#define LDS_AS __attribute__((address_space(3)))

// One 1 KB global -> LDS load: lane i's 16 bytes at sbase + voff land at LDS byte address
// lds + 16i.  Issued from inline assembly, so the compiler neither counts it nor waits for
// it; the kernel waits (vmcnt) before the barrier that publishes a tile.  M0 carries the
// LDS address and needs one wait state before the load.  sbase and lds are wave-uniform.
// M0 is a reserved register; these kernels use it nowhere else (each statement sets it
// right before its load), so the clobber only keeps the compiler from assuming it intact.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
    // readfirstlane returns int: widen through uint32_t, never by sign extension
    const uint64_t a = reinterpret_cast<uint64_t>(sbase);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const char* base = reinterpret_cast<const char*>(((uint64_t)hi << 32) | (uint64_t)lo);
    const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 : : "v"(voff), "s"(base), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read: each 16 lanes read a 4-row x 16-column block of 16-bit elements;
// lane L supplies the address of row (L%16)/4, columns 4(L%4)..4(L%4)+3, and receives
// column L%16, rows 0..3.
__device__ __forceinline__ bf16x4 read_tr(const LDS_AS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
}

// System-scope (write-through, uncached) 16-byte accesses for the stream-K workspace: a
// completed store is in memory, where a workgroup on any XCD reads it, so no cache
// maintenance is needed.  A load statement issues its loads and waits for them itself,
// so its outputs are valid when it ends (the compiler does not track these loads).
// OFF is an immediate byte offset (< 4096) from p.
template <int OFF>
__device__ __forceinline__ void store_sys(float* p, f32x4 x) {
    asm volatile("global_store_dwordx4 %0, %1, off offset:%2 sc0 sc1" : : "v"(p), "v"(x), "i"(OFF) : "memory");
}
__device__ __forceinline__ f32x4 load_sys(const float* p) {
    f32x4 x;
    asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(x) : "v"(p) : "memory");
    return x;
}
// four 16-byte loads at p, p + 1 KB, p + 2 KB, p + 3 KB
__device__ __forceinline__ void load_sys4(const float* p, f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
    asm volatile("global_load_dwordx4 %0, %4, off sc0 sc1\n\t"
                 "global_load_dwordx4 %1, %4, off offset:1024 sc0 sc1\n\t"
                 "global_load_dwordx4 %2, %4, off offset:2048 sc0 sc1\n\t"
                 "global_load_dwordx4 %3, %4, off offset:3072 sc0 sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d) : "v"(p) : "memory");
}

// ACCUM: continue from a previous result (o_prev, lse_prev) over other keys instead of
// starting afresh; o and lse may then be the very arrays o_prev and lse_prev (each
// element is read before it is written, by the same lane), so none of them is restrict.
// SPLIT = false: one whole tile per workgroup, tiles [tile_base, tile_base + grid).
// SPLIT = true: the split part, tiles from tile_base on, as stream-K unit ranges.
// KG = 2 (8 waves, whole tiles only): two groups of 4 waves take the same 128 query rows
// and each half of the tile's key blocks, with key tiles of their own in LDS; group 1
// hands its state to group 0 through LDS at the end.  For grids of at most one tile per
// CU (a Ring round over a short Q block) this puts 8 waves on every busy CU instead of 4.
template <int D, int NW, int KG, bool OUT_F32, bool ACCUM, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 8 / NW)
void attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, void* o, float* lse,
                     const float* o_prev, const float* lse_prev,
                     int Nq, int Nkv, int H, int q_batches, int kv_chunks, float scale_log2,
                     int n_qtiles, int tile_base, StreamK work) {
    static_assert(KG == 1 || (NW == 8 && !SPLIT), "key groups: 8-wave whole tiles");
    constexpr int kThreads = NW * 64;
    constexpr int kGW = NW / KG;         // waves per key group
    constexpr int kBlockM = kGW * 32;    // query rows per workgroup
    using L = TileLayout<D, kGW>;
    // LDS: K and V tiles, two buffers each ([K0 | K1 | V0 | V1], key-major, layout in
    // TileLayout) during the key loop; the output tile on its way to memory after it.
    constexpr int kStageBytes = kBlockM * (4 * D + 16) + kBlockM * 4;   // f32 output staging
    constexpr int kTilesBytes = KG * 4 * L::kTileBytes;                   // each group: K0 K1 V0 V1
    constexpr int kLdsBytes = kTilesBytes > kStageBytes ? kTilesBytes : kStageBytes;
    __shared__ __attribute__((aligned(16))) char s_lds[kLdsBytes];
    __shared__ int s_ready;
    auto lds_addr = [&](const char* p) { return (uint32_t)(size_t)(const LDS_AS void*)p; };

    const int tid = threadIdx.x;
    const int wave_all = tid >> 6;
    const int kg = wave_all / kGW;          // key group (0 with KG = 1)
    const int wave = wave_all % kGW;        // wave within the group: query rows 32 wave + r
    const int lane = tid & 63;
    const int g = lane >> 5;   // lane half
    const int r = lane & 31;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    char* const s_tiles = s_lds + __builtin_amdgcn_readfirstlane(kg) * 4 * L::kTileBytes;
    auto sK = [&](int buf) { return s_tiles + buf * L::kTileBytes; };
    auto sV = [&](int buf) { return s_tiles + (2 + buf) * L::kTileBytes; };

    const int tok_stride = H * D;  // elements between consecutive tokens (H*D <= 2^24, checked on the host)
    const long ts_bytes = 2L * tok_stride;

    // Per-lane load offsets (bytes from a tile's first key), fixed for the whole kernel:
    // load instruction i of this wave fetches the piece TileLayout assigns to this lane.
    // A tile spans 64 * ts_bytes < 2^31 bytes, so they fit 32 bits.
    constexpr int NL = L::kLoadsPerWave;
    uint32_t k_src[NL], v_src[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        k_src[i] = (uint32_t)(L::k_src_key(wave, i, lane) * ts_bytes + 16 * L::k_src_chunk(wave, i, lane));
        v_src[i] = (uint32_t)(L::v_src_key(wave, i, lane) * ts_bytes + 16 * L::v_src_chunk(wave, i, lane));
    }

    // the current tile's coordinates and state
    const uint16_t* kbase = k;
    const uint16_t* vbase = v;
    int b = 0, h = 0, qrow = 0;
    bf16x8 qf[D / 16];
    f32x16 acc[D / 32];
    float m_run;   // reference max of this lane's query row (log2 units)
    float l_run;   // this lane's half of the row sum, relative to m_run

    // Global -> LDS for the tile starting at key kv0 into buffer buf.  The ragged last tile
    // repeats its last key for rows past Nkv (finite values: their logits are masked and
    // their weights are 0).
    auto load_tile = [&](auto partial_c, int kv0, int buf) {
        constexpr bool PARTIAL = decltype(partial_c)::value;
        const char* kt = reinterpret_cast<const char*>(kbase) + kv0 * ts_bytes;
        const char* vt = reinterpret_cast<const char*>(vbase) + kv0 * ts_bytes;
        const uint32_t kd = lds_addr(sK(buf)), vd = lds_addr(sV(buf));
        const int last = Nkv - 1 - kv0;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            uint32_t ko = k_src[i], vo = v_src[i];
            if constexpr (PARTIAL) {
                ko = (uint32_t)(min(L::k_src_key(wave, i, lane), last) * ts_bytes + 16 * L::k_src_chunk(wave, i, lane));
                vo = (uint32_t)(min(L::v_src_key(wave, i, lane), last) * ts_bytes + 16 * L::v_src_chunk(wave, i, lane));
            }
            dma16(kt, ko, kd + L::load_block(wave_u, i));
            dma16(vt, vo, vd + L::load_block(wave_u, i));
        }
    };
    using FULL = std::false_type;
    using PARTIAL = std::true_type;

    // Weights of one 32-key half against the current reference max m_run: exp2(s*c - m_run)
    // rounded to bf16 for the P.V product; returns the f32 sum of this lane's 16 rounded
    // weights.  The row sum is taken over the rounded weights, two per v_dot2 against (1, 1):
    // numerator (P.V on the bf16 P) and denominator then round the same way.
    auto half_weights = [&](const f32x16& s, bf16x8 (&pf)[2]) -> float {
        float lsum = 0.f;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            f32x8 e;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e[i] = __builtin_amdgcn_exp2f(fmaf(s[hf * 8 + i], scale_log2, -m_run));
            pf[hf] = __builtin_convertvector(e, bf16x8);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[hf], pf[hf], 0, 1), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[hf], pf[hf], 2, 3), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[hf], pf[hf], 4, 5), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[hf], pf[hf], 6, 7), ones, lsum, false);
        }
        return lsum;
    };

    // Online-softmax update for one 32-key half of a tile.  The weights are first taken
    // against the current reference max.  They are non-negative, so when every lane's sum of
    // its 16 weights is at most 2^kRescaleThreshold, so is every weight: the reference stays
    // and no row max is formed (the common case once a row's larger logits have been seen).
    // Otherwise (a larger weight, or the +inf / NaN weights of a row's first half, whose
    // reference is still -inf) the reference moves to kHeadroom above the half's row max, the
    // accumulators need the rescale by alpha, and the weights are taken again.  Returns whether the rescale
    // is needed (wave-uniform); lsum is the f32 sum of this lane's 16 rounded weights.
    auto softmax_half = [&](const f32x16& s, bf16x8 (&pf)[2], float& lsum, float& alpha) -> bool {
        lsum = half_weights(s, pf);
        alpha = 1.0f;
        // compared as bit patterns: a non-negative float orders like its bits, and +inf and
        // the NaNs lie above every finite bound (the kernel is built without NaN semantics)
        if (__all(__float_as_uint(lsum) <= __float_as_uint(kMaxLaneSum))) return false;
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float m_new = fmaxf(m_run, halves_max(mx) * scale_log2 + kHeadroom);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 from a -inf reference, 1 if unchanged
        m_run = m_new;
        l_run *= alpha;
        lsum = half_weights(s, pf);
        return true;
    };
    auto rescale_acc = [&](float alpha) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    };
    auto s_half = [&](f32x16& s, const LDS_AS char* sk, int kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 a = *reinterpret_cast<const LDS_AS bf16x8*>(sk + L::k_frag(kb, ks, lane));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
        }
    };
    auto pv_half = [&](const bf16x8 (&pf)[2], const LDS_AS char* sv, int kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x4 lo = read_tr(sv + L::v_frag(kb, hf, db, 0, lane));
                const bf16x4 hi = read_tr(sv + L::v_frag(kb, hf, db, 1, lane));
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[hf], acc[db], 0, 0, 0);
            }
    };

    // One key tile, as four blocks that each pair MFMAs with VALU work independent of them,
    // so a wave keeps its softmax under its own MFMAs:
    //   S of key half 0
    //   S of key half 1            with  the softmax of half 0
    //   P.V of half 0              with  the softmax of half 1
    //   P.V of half 1
    // Meanwhile the next tile (PF: 0 none, 1 a full tile, 2 the ragged last tile) travels
    // into the other buffer; the wait for it sits right before the closing barrier.
    auto step = [&](auto pf_c, auto mask_c, int it) {
        constexpr int PF = decltype(pf_c)::value;
        constexpr bool MASK = decltype(mask_c)::value;
        const int buf = it & 1;
        const int kv0 = it * kBlockN;

        const LDS_AS char* sk = (const LDS_AS char*)(const LDS_AS void*)sK(buf);
        const LDS_AS char* sv = (const LDS_AS char*)(const LDS_AS void*)sV(buf);
        f32x16 s0, s1;
        bf16x8 p0[2], p1[2];
        float ls0, ls1, a0, a1;

        s_half(s0, sk, 0);
        __builtin_amdgcn_sched_barrier(0);
        // the next tile goes into the other buffer, which the previous step's barrier freed;
        // issued after the first block's MFMAs rather than before them (0.5% faster at long
        // key ranges, 4% at 512 keys)
        if constexpr (PF == 1) load_tile(FULL{}, kv0 + kBlockN, buf ^ 1);
        if constexpr (PF == 2) load_tile(PARTIAL{}, kv0 + kBlockN, buf ^ 1);
        // All blocks run at equal wave priority.  (Raising it for the two softmax blocks was
        // 1-2% faster while they formed a row max every half; with the lighter lane-sum
        // softmax it is 1.6-2.2% slower at long key ranges.)
        s_half(s1, sk, 1);
        if constexpr (MASK) {  // keys past the end get weight 0
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kv0 + 16 * (i / 8) + 8 * g + (i % 8);
                if (key >= Nkv) s0[i] = -INFINITY;
            }
        }
        const bool r0 = softmax_half(s0, p0, ls0, a0);
        asm volatile("" : "+v"(p0[0]), "+v"(p0[1]), "+v"(ls0));   // keep it in this block
        __builtin_amdgcn_sched_barrier(0);
        if (r0) rescale_acc(a0);
        pv_half(p0, sv, 0);
        if constexpr (MASK) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kv0 + 32 + 16 * (i / 8) + 8 * g + (i % 8);
                if (key >= Nkv) s1[i] = -INFINITY;
            }
        }
        const bool r1 = softmax_half(s1, p1, ls1, a1);
        asm volatile("" : "+v"(p1[0]), "+v"(p1[1]), "+v"(ls1));
        __builtin_amdgcn_sched_barrier(0);
        l_run += ls0 * a1 + ls1;
        if (r1) rescale_acc(a1);
        pv_half(p1, sv, 1);
        __builtin_amdgcn_sched_barrier(0);   // the P.V MFMAs issue before the wait
        if constexpr (PF != 0) wait_dma();
        __syncthreads();
    };
    using PF0 = std::integral_constant<int, 0>;
    using PF1 = std::integral_constant<int, 1>;
    using PF2 = std::integral_constant<int, 2>;
    using NOMASK = std::integral_constant<bool, false>;
    using MASKED = std::integral_constant<bool, true>;

    // Key tiles [lo, hi) of the current query tile, continuing the running state.  With
    // KG = 2, group 0 takes the first ceil(n/2) of them and group 1 the rest; both pass the
    // same barriers (group 1 one extra when it has one tile fewer).
    auto run = [&](int lo_all, int hi_all) {
        int lo = lo_all, hi = hi_all;
        if constexpr (KG == 2) {
            const int mid = lo_all + (hi_all - lo_all + 1) / 2;
            if (kg == 0) hi = mid;
            else lo = mid;
        }
        const bool has_tail = hi > lo && hi == work.n_kv && Nkv % kBlockN != 0;  // the ragged last tile
        const int n_full = (has_tail ? hi - 1 : hi) - lo;
        if (n_full > 0) load_tile(FULL{}, lo * kBlockN, lo & 1);
        else if (has_tail) load_tile(PARTIAL{}, lo * kBlockN, lo & 1);
        wait_dma();
        // the Q loads are complete too: tell the compiler, which does not see the tile
        // loads, so that it puts no wait for them inside the key loop
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int it = lo;
        for (; it + 1 < lo + n_full; ++it) step(PF1{}, NOMASK{}, it);
        if (n_full > 0) {
            if (has_tail) step(PF2{}, NOMASK{}, it);
            else step(PF0{}, NOMASK{}, it);
            ++it;
        }
        if (has_tail) step(PF0{}, MASKED{}, it);
        if constexpr (KG == 2) {
            if (hi - lo < (hi_all - lo_all + 1) / 2) __syncthreads();   // group 1's missing step
            // group 1 hands its state to group 0 (same rows, other keys) through LDS, which
            // the key tiles no longer need: [wave][acc 16 x D/32 + m, l][lane]
            float* xs = reinterpret_cast<float*>(s_lds) + wave * ((D / 2) + 2) * 64 + lane;
            if (kg == 1) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xs[(db * 16 + i) * 64] = acc[db][i];
                xs[(D / 2) * 64] = m_run;
                xs[(D / 2 + 1) * 64] = l_run;
            }
            __syncthreads();
            if (kg == 0) {
                const float m_oth = xs[(D / 2) * 64];
                const float m_new = fmaxf(m_run, m_oth);   // finite: group 0 saw at least one key
                const float f_own = __builtin_amdgcn_exp2f(m_run - m_new);
                const float f_oth = __builtin_amdgcn_exp2f(m_oth - m_new);   // 0 for a group without keys
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[db][i] = acc[db][i] * f_own + xs[(db * 16 + i) * 64] * f_oth;
                l_run = l_run * f_own + xs[(D / 2 + 1) * 64] * f_oth;
                m_run = m_new;
            }
            __syncthreads();   // LDS is free again
        }
    };

    // Sets the coordinates of query tile `tile`, loads its Q^T fragments (held for the
    // whole key loop) and clears the running state.
    auto begin_tile = [&](int tile) {
        const int qt = tile % n_qtiles;
        const int bh = tile / n_qtiles;
        h = bh % H;
        b = bh / H;                              // output batch: chunk-major (t * q_batches + bq)
        const int bq = b % q_batches;            // the query batch
        const long bkv = (long)bq * kv_chunks + b / q_batches;   // its key chunk, Nkv keys long
        kbase = k + (bkv * Nkv * H + h) * D;
        vbase = v + (bkv * Nkv * H + h) * D;
        qrow = qt * kBlockM + wave * 32 + r;
        const uint16_t* qp = q + (((long)bq * Nq + qrow) * H + h) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 x = qrow < Nq ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
        m_run = -INFINITY;
        l_run = 0.f;
    };

    // O = acc / l and LSE = m + log2(l) (natural log of the scaled logits), or with ACCUM
    // the combination with the previous result.  O goes out through LDS, which the key
    // loop no longer needs: each lane leaves its 4-column pieces of its row there, then
    // every store instruction writes whole rows (16 bytes per thread, consecutive threads
    // along a row) instead of 8- or 16-byte pieces of 32 rows.  With ACCUM the tile is
    // staged in f32, so that the combination rounds once.
    auto finish_tile = [&]() {
        constexpr bool STAGE_F32 = OUT_F32 || ACCUM;
        constexpr int ES = STAGE_F32 ? 4 : 2;            // staged element bytes
        constexpr int RS = D * ES + 16;                  // staged row stride (bytes), padded
        constexpr int OES = OUT_F32 ? 4 : 2;             // output element bytes
        constexpr int EPC = 16 / OES;                    // output elements per 16-byte chunk
        constexpr int CPR = D / EPC;                     // chunks per row
        static_assert(kBlockM * RS + kBlockM * 4 <= (int)sizeof(s_lds), "output tile fits in LDS");
        char* st = s_lds;
        float* s_wprev = reinterpret_cast<float*>(st + kBlockM * RS);
        const int lrow = wave * 32 + r;                  // this lane's row in the tile
        // with KG = 2 group 0 holds the whole result (group 1 folded into it)
        const bool owner = KG == 1 || kg == 0;
        const float l_tot = halves_sum(l_run);
        float w_cur = 1.0f / l_tot, w_prev = 0.0f;
        if (owner && qrow < Nq) {
            const long lidx = ((long)b * H + h) * Nq + qrow;
            const float lse_cur = (m_run + log2f(l_tot)) * 0.693147180559945309f;
            float lse_out = lse_cur;
            if constexpr (ACCUM) {
                // L = ln(e^lse_prev + e^lse_cur); o = e^(lse_prev - L) o_prev + e^(lse_cur - L) o_cur
                // (the across-rounds accumulation of Ring attention).  lse_prev = -inf holds no
                // keys: its o_prev is not read.
                const float lp = lse_prev[lidx];
                if (lp != -INFINITY) {
                    const float mx = fmaxf(lp, lse_cur);
                    const float ep = __expf(lp - mx), ec = __expf(lse_cur - mx);
                    const float inv = 1.0f / (ep + ec);
                    w_prev = ep * inv;
                    w_cur *= ec * inv;
                    lse_out = mx + __logf(ep + ec);
                }
            }
            if (g == 0) lse[lidx] = lse_out;
        }
        // the key loop's last step ended with a barrier: LDS is free
        if (owner) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 x = {acc[db][4 * i4] * w_cur, acc[db][4 * i4 + 1] * w_cur,
                                     acc[db][4 * i4 + 2] * w_cur, acc[db][4 * i4 + 3] * w_cur};
                    char* dst = st + lrow * RS + (db * 32 + 8 * i4 + 4 * g) * ES;
                    if constexpr (STAGE_F32) *reinterpret_cast<f32x4*>(dst) = x;
                    else *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(x, bf16x4);
                }
            if constexpr (ACCUM) {
                if (g == 0) s_wprev[lrow] = w_prev;
            }
        }
        __syncthreads();
        const int row0 = qrow - lrow;                    // the tile's first query row
#pragma unroll 4
        for (int idx = tid; idx < kBlockM * CPR; idx += kThreads) {
            const int row = idx / CPR, c = idx - (idx / CPR) * CPR;
            if (row0 + row >= Nq) continue;
            const long off = (((long)b * Nq + row0 + row) * H + h) * D + c * EPC;   // elements
            const char* src = st + row * RS + c * EPC * ES;
            if constexpr (!STAGE_F32) {
                *reinterpret_cast<u32x4*>(static_cast<__bf16*>(o) + off) = *reinterpret_cast<const u32x4*>(src);
            } else if constexpr (OUT_F32) {
                f32x4 x = *reinterpret_cast<const f32x4*>(src);
                if constexpr (ACCUM) {
                    const float wp = s_wprev[row];
                    if (wp != 0.0f) x += wp * *reinterpret_cast<const f32x4*>(o_prev + off);
                }
                *reinterpret_cast<f32x4*>(static_cast<float*>(o) + off) = x;
            } else {   // ACCUM into a bf16 output: 8 values per chunk
                f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
                f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 16);
                const float wp = s_wprev[row];
                if (wp != 0.0f) {
                    x0 += wp * *reinterpret_cast<const f32x4*>(o_prev + off);
                    x1 += wp * *reinterpret_cast<const f32x4*>(o_prev + off + 4);
                }
                const f32x8 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(o) + off) = __builtin_convertvector(x, bf16x8);
            }
        }
        __syncthreads();   // LDS holds key tiles again after this
    };

    if constexpr (!SPLIT) {
        // Whole tiles, one resident workgroup per slot: workgroup g takes tiles g, g + grid,
        // ... in XCD-contiguous order (with the GPU's slot counts, 512 or 256, grid is a
        // multiple of 8 whenever a workgroup takes more than one tile, so its tiles stay on
        // its XCD).  The next tile's coordinates and Q
        // loads go out before this tile's epilogue, which hides their latency (FLUX: 1.3%
        // faster than one workgroup per tile).
        const int total = work.n_dp;
        int t = blockIdx.x;
        if (t < total) begin_tile(xcd_contiguous(t, total) + tile_base);
        while (t < total) {
            run(0, work.n_kv);
            const int tn = t + (int)gridDim.x;
            int nb = b, nh = h, nqrow = qrow;
            const uint16_t* nkb = kbase;
            const uint16_t* nvb = vbase;
            if (tn < total) {   // as begin_tile, into separate coordinates (qf is free now)
                const int tile = xcd_contiguous(tn, total) + tile_base;
                const int qt = tile % n_qtiles;
                const int bh = tile / n_qtiles;
                nh = bh % H;
                nb = bh / H;
                const int bq = nb % q_batches;
                const long bkv = (long)bq * kv_chunks + nb / q_batches;
                nkb = k + (bkv * Nkv * H + nh) * D;
                nvb = v + (bkv * Nkv * H + nh) * D;
                nqrow = qt * kBlockM + wave * 32 + r;
                const uint16_t* qp = q + (((long)bq * Nq + nqrow) * H + nh) * D + 8 * g;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    u32x4 x = nqrow < Nq ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
                    qf[ks] = __builtin_bit_cast(bf16x8, x);
                }
            }
            finish_tile();
            b = nb;
            h = nh;
            qrow = nqrow;
            kbase = nkb;
            vbase = nvb;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
            m_run = -INFINITY;
            l_run = 0.f;
            t = tn;
        }
        return;
    } else {
        // The workspace is written and read with system-scope (write-through, uncached)
        // accesses, so no cache maintenance is needed: once a workgroup's stores have
        // completed they are in memory, where every XCD reads them.
        const int wg = xcd_contiguous(blockIdx.x, work.G_sk);
        // this launch's flag value (streamk.h); the launch count changes only after the
        // launch, so every workgroup reads the same one
        const unsigned long long flag_val = work.flag == nullptr ? 0ull :
            sk_flag_value(work.epoch, __hip_atomic_load(work.launch_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
        long u = sk_first_unit(work, wg);
        const long u_end = sk_first_unit(work, wg + 1);
        while (u < u_end) {
            const int st = (int)(u / work.n_kv);
            const long tile_u0 = (long)st * work.n_kv;
            const int lo = (int)(u - tile_u0);
            const int hi = (int)((u_end < tile_u0 + work.n_kv ? u_end : tile_u0 + work.n_kv) - tile_u0);
            u = tile_u0 + hi;
            begin_tile(tile_base + st);
            // one run of key tiles per pass; a finaliser whose helpers have not published
            // in time takes a second pass over the rest of the tile
            int seg_lo = lo, seg_hi = hi;
            bool publish = false;
            for (;;) {
                run(seg_lo, seg_hi);
                if (lo > 0) { publish = true; break; }
                if (seg_hi == work.n_kv) break;
                // the tile's finaliser: fold in the states of the owners of keys [hi, n_kv)
                const int g_first = sk_owner(work, tile_u0 + hi);
                const int g_last = sk_owner(work, tile_u0 + work.n_kv - 1);
                if (tid == 0) {
                    // the helpers run concurrently and finish their pieces about now: poll,
                    // but only for a bounded time
                    int ok = 0;
                    for (int poll = 0; poll < work.max_polls && !ok; ++poll) {
                        ok = 1;
                        for (int gg = g_first; gg <= g_last; ++gg)
                            ok &= __hip_atomic_load(work.flag + gg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == flag_val;
                        if (!ok) __builtin_amdgcn_s_sleep(8);
                    }
                    s_ready = ok;
                }
                __syncthreads();
                const bool ready = s_ready != 0;
                __syncthreads();   // s_ready is rewritten by the next finaliser check
                if (!ready) {      // not published in time: compute the rest here
                    seg_lo = seg_hi;
                    seg_hi = work.n_kv;
                    continue;
                }
                for (int gg = g_first; gg <= g_last; ++gg) {
                    const float* wa = work.ws_acc + ((long)gg * kThreads + wave * 64) * (D / 2) + lane * 4;
                    const f32x4 ml = load_sys(work.ws_ml + ((long)gg * kThreads + tid) * 4);
                    const float m_new = fmaxf(m_run, ml[0]);
                    const float f_own = __builtin_amdgcn_exp2f(m_run - m_new);
                    const float f_oth = __builtin_amdgcn_exp2f(ml[0] - m_new);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {   // one 32-column block at a time
                        f32x4 x[4];
                        load_sys4(wa + db * 1024, x[0], x[1], x[2], x[3]);
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            acc[db][i] = acc[db][i] * f_own + x[i / 4][i % 4] * f_oth;
                    }
                    l_run = l_run * f_own + ml[1] * f_oth;
                    m_run = m_new;
                }
                break;
            }
            if (publish) {
                // not the tile's first keys: hand the raw state to the tile's finaliser
                // slot layout [wave][store j][lane][4]: each store instruction writes 1 KB
                float* wa = work.ws_acc + ((long)wg * kThreads + wave * 64) * (D / 2) + lane * 4;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    float* wb = wa + db * 1024;   // 4 stores of 1 KB from here
                    store_sys<0>(wb, __builtin_shufflevector(acc[db], acc[db], 0, 1, 2, 3));
                    store_sys<1024>(wb, __builtin_shufflevector(acc[db], acc[db], 4, 5, 6, 7));
                    store_sys<2048>(wb, __builtin_shufflevector(acc[db], acc[db], 8, 9, 10, 11));
                    store_sys<3072>(wb, __builtin_shufflevector(acc[db], acc[db], 12, 13, 14, 15));
                }
                const f32x4 ml = {m_run, l_run, 0.f, 0.f};
                store_sys<0>(work.ws_ml + ((long)wg * kThreads + tid) * 4, ml);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's stores are done
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(work.flag + wg, flag_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                continue;
            }
            finish_tile();
        }
    }
}

template <int D, int NW, int KG, bool OUT_F32, bool ACCUM, bool SPLIT>
void launch_one(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, float* lse,
                const float* o_prev, const float* lse_prev, int Nq, int Nkv, int H, int qb,
                int kvc, float scale_log2, int n_qtiles, int grid, int tile_base,
                const StreamK& work, hipStream_t stream) {
    attn_fwd_kernel<D, NW, KG, OUT_F32, ACCUM, SPLIT><<<dim3(grid), dim3(NW * 64), 0, stream>>>(
        q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, tile_base, work);
}

template <int D, int NW, int KG, bool SPLIT>
void launch_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, float* lse,
              const float* o_prev, const float* lse_prev, int Nq, int Nkv, int H, int qb,
              int kvc, float scale_log2, int n_qtiles, int grid, int tile_base,
              const StreamK& work, bool out_f32, hipStream_t stream) {
    const bool accum = o_prev != nullptr;
    if (out_f32) {
        if (accum) launch_one<D, NW, KG, true, true, SPLIT>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, grid, tile_base, work, stream);
        else launch_one<D, NW, KG, true, false, SPLIT>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, grid, tile_base, work, stream);
    } else {
        if (accum) launch_one<D, NW, KG, false, true, SPLIT>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, grid, tile_base, work, stream);
        else launch_one<D, NW, KG, false, false, SPLIT>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, grid, tile_base, work, stream);
    }
}

// Advances a split workspace's launch count (streamk.h), after the split launch that read it.
__global__ __launch_bounds__(64) void advance_launch_count_kernel(unsigned long long* ctr) {
    if (threadIdx.x == 0) {
        const unsigned long long n = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(ctr, n + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// the launches of one schedule: whole tiles first (complete rounds of the slots), then the
// split part
template <int D, int NW, int KG>
void launch_schedule(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, float* lse,
                     const float* o_prev, const float* lse_prev, int Nq, int Nkv, int H, int qb,
                     int kvc, float scale_log2, int n_qtiles, const StreamK& work, bool out_f32,
                     hipStream_t stream) {
    if (work.n_dp > 0)   // at most one workgroup per slot (persistent over the whole tiles)
        launch_d<D, NW, KG, false>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles,
                                   work.n_dp < work.slots ? work.n_dp : work.slots, 0, work, out_f32, stream);
    if constexpr (KG == 1) {
        if (work.G_sk > 0) {
            launch_d<D, NW, KG, true>(q, k, v, o, lse, o_prev, lse_prev, Nq, Nkv, H, qb, kvc, scale_log2, n_qtiles, work.G_sk, work.n_dp, work, out_f32, stream);
            if (work.launch_ctr != nullptr) advance_launch_count_kernel<<<1, 64, 0, stream>>>(work.launch_ctr);
        }
    }
}

// Static workspace of attn_fwd_lse_noalloc: the states and flags of the split pieces, for
// callers that may not allocate.  Sized for the largest split part on a 256-CU MI355X
// (at most 512 workgroups of 256 threads or 256 of 512, 64 f32 accumulators and 4 f32 of
// running max and sum per thread at head_dim 128, and one 8-byte flag per workgroup);
// a schedule needing more is rejected before launch.  Each device holds its own copy
// until the process ends.  In host code `scratch` only names the symbol: its device
// address comes from hipGetSymbolAddress (DeviceInfo::scratch).
constexpr size_t kScratchBytes = 36u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Per-device launch facts: compute units, the address of this device's copy of
// `scratch`, and (created at the first call that needs it) a memory pool for the
// stream-ordered workspace.
struct DeviceInfo {
    int cus = 0;
    char* scratch = nullptr;
    hipError_t scratch_err = hipSuccess;
    hipMemPool_t pool = nullptr;
};

// Sets *out to the current device's facts, gathering them on its first call there (with
// that device current).  With want_pool, also creates the device's pool if it has none.
hipError_t device_info(DeviceInfo** out, bool want_pool) {
    static std::mutex mu;
    static DeviceInfo infos[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    DeviceInfo& d = infos[dev];
    if (d.cus == 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        void* p = nullptr;
        d.scratch_err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.scratch = d.scratch_err == hipSuccess ? static_cast<char*>(p) : nullptr;
        d.cus = cus;
    }
    if (want_pool && d.pool == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;   // keep freed workspace in the pool for the next call
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            hipMemPoolDestroy(pool);
            return e;
        }
        d.pool = pool;
    }
    *out = &d;
    return hipSuccess;
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           const float* o_prev, const float* lse_prev, int B, int Nq, int Nkv,
                           int H, int D, int P, float scale, bool out_f32, bool static_ws,
                           bool* ws_too_small, hipStream_t stream) {
    // P > 1: P equal key chunks of Nkv / P keys each, one result per (chunk, batch), as
    // if the chunks were P * B batches sharing the batch's queries
    const int Bq = B;
    B *= P;
    Nkv /= P;
    if (ws_too_small != nullptr) *ws_too_small = false;
    DeviceInfo* dev = nullptr;
    hipError_t e = device_info(&dev, false);
    if (e != hipSuccess) return e;
    // DTL_ATTN_SLOTS (tests, tuning) schedules as if the GPU held that many workgroups; it
    // changes which tiles are split, never the result.  It may only lower the count.
    const int n_kv = (Nkv + kBlockN - 1) / kBlockN;
    // 8-wave workgroups (256-row tiles, one per CU) for key ranges of more than 16 blocks
    // whose 128-row tiles would be more than one per CU; 4-wave ones (128 rows, two per CU)
    // otherwise.  Measured on full grids (27280 queries, 24 heads), 8 waves take 1.027x the
    // 4-wave time at 8 key blocks, 1.011x at 12, 1.000x at 16, 0.966x at 24 and 32, 0.978x
    // at 48; 0.924x at 4608 x 1152 and 0.962x for the FLUX Ring-4 share's four chunks in one
    // launch.  Between one and two 128-row tiles per CU some CU runs two of them, which takes
    // longer than one 256-row tile even with CUs left idle: 0.89-0.93x at 2304 x 4608,
    // 3072 x 4608 (16 heads), 1536 x 27280, 2560 x 2048 and 4608 x 4608 (12 heads).
    bool wide = D == 128 && n_kv > 16 && (long)((Nq + 127) / 128) * H * B > dev->cus;
    // DTL_ATTN_WAVES (tests, tuning) = 4 or 8 picks the workgroup size for head_dim 128;
    // like DTL_ATTN_SLOTS it changes the schedule, never the result
    if (const char* env = getenv("DTL_ATTN_WAVES")) {
        const long want = strtol(env, nullptr, 10);
        if (D == 128 && (want == 4 || want == 8)) wide = want == 8;
    }
    // Two key groups per 8-wave workgroup (128-row tiles, one workgroup per CU) when the
    // 128-row tiles are at most one per CU, so that every busy CU runs 8 waves rather than
    // 4 (a Ring round over a short Q block: the FLUX Ring-4 share's 1152-row block is 216
    // tiles).  DTL_ATTN_KEYSPLIT (tests, tuning) = 0 or 1 turns it off or on wherever it
    // applies (head_dim 128, 128-row tiles, at least 2 key blocks); never a different result
    // beyond rounding order.
    const bool ks_ok = !wide && D == 128 && n_kv >= 2;
    bool keysplit = ks_ok && (long)((Nq + 127) / 128) * H * B <= dev->cus;
    if (const char* env = getenv("DTL_ATTN_KEYSPLIT")) keysplit = ks_ok && strtol(env, nullptr, 10) != 0;
    const int nw = wide || keysplit ? 8 : 4;
    const int kgr = keysplit ? 2 : 1;
    const int rows = 32 * nw / kgr;   // query rows per tile
    long slots = (long)(8 / nw) * dev->cus;
    if (const char* env = getenv("DTL_ATTN_SLOTS")) {
        const long want = strtol(env, nullptr, 10);
        if (want > 0 && want < slots) slots = want;
    }
    const int n_qtiles = (Nq + rows - 1) / rows;
    const long tiles = (long)n_qtiles * H * B;   // the caller has checked that this fits an int
    // Split only where whole tiles would leave most of the GPU idle (streamk.h).  A larger
    // remainder already runs well as whole tiles: with fewer workgroups than slots many
    // CUs hold a single workgroup, whose waves then run faster (measured: 1.2x per
    // workgroup), while every split piece pays a pipeline start, a publish and a merge, and
    // the split part a second launch; with few key blocks per tile (cross-attention's 512
    // keys) those costs exceed the idle tail.
    // DTL_ATTN_SPLIT (tests, tuning) = 0 or 1: never split, or split any remainder; like the
    // variables above it changes who computes which keys, never the result
    int force_split = -1;
    if (const char* env = getenv("DTL_ATTN_SPLIT")) force_split = strtol(env, nullptr, 10) != 0 ? 1 : 0;
    StreamK work = plan_stream_k(tiles, n_kv, slots, force_split);
    if (keysplit) {   // whole tiles only
        work.n_dp = (int)tiles;
        work.G_sk = 0;
    }
    work.slots = (int)slots;
    // DTL_ATTN_MAX_POLLS (tests) lowers the finalisers' wait for their helpers; at 0 each
    // finaliser computes the rest of its tile itself.  Like the two variables above it
    // changes who computes which keys, never the result.
    work.max_polls = kMaxPolls;
    if (const char* env = getenv("DTL_ATTN_MAX_POLLS")) {
        const long want = strtol(env, nullptr, 10);
        if (want >= 0 && want < kMaxPolls) work.max_polls = (int)want;
    }
    // a workspace is needed only when some split range starts inside a tile
    bool split = false;
    for (int gg = 1; gg < work.G_sk && !split; ++gg) split = sk_first_unit(work, gg) % work.n_kv != 0;
    void* ws = nullptr;   // pool workspace of this call, freed after its kernels
    if (split) {
        // Flags are compared with this launch's flag value (streamk.h), so no workspace needs
        // clearing: whatever an earlier launch, an earlier replay of a captured launch, or
        // no launch left there never matches.  Layout: [launch count, 16 B | acc | ml | flags].
        static std::atomic<unsigned long long> epochs{0x9E3779B97F4A7C15ull};
        const size_t ctr_bytes = 16;
        const size_t acc_bytes = (size_t)work.G_sk * (nw * 64) * (D / 2) * sizeof(float);
        const size_t ml_bytes = (size_t)work.G_sk * (nw * 64) * 4 * sizeof(float);
        const size_t flag_bytes = (size_t)work.G_sk * sizeof(unsigned long long);
        const size_t need = ctr_bytes + acc_bytes + ml_bytes + flag_bytes;
        char* base = nullptr;
        if (static_ws) {
            if (dev->scratch == nullptr) return dev->scratch_err != hipSuccess ? dev->scratch_err : hipErrorInvalidSymbol;
            if (need > kScratchBytes) {
                if (ws_too_small != nullptr) *ws_too_small = true;
                return hipErrorInvalidValue;
            }
            base = dev->scratch;
        } else {
            e = device_info(&dev, true);
            if (e != hipSuccess) return e;
            e = hipMallocFromPoolAsync(&ws, need, dev->pool, stream);
            if (e != hipSuccess) return e;
            base = static_cast<char*>(ws);
        }
        work.launch_ctr = reinterpret_cast<unsigned long long*>(base);
        work.ws_acc = reinterpret_cast<float*>(base + ctr_bytes);
        work.ws_ml = reinterpret_cast<float*>(base + ctr_bytes + acc_bytes);
        work.flag = reinterpret_cast<unsigned long long*>(base + ctr_bytes + acc_bytes + ml_bytes);
        work.epoch = epochs.fetch_add(1) + 1;
    }
    const float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    auto qq = static_cast<const uint16_t*>(q);
    auto kk = static_cast<const uint16_t*>(k);
    auto vv = static_cast<const uint16_t*>(v);
    if (D == 128 && wide)
        launch_schedule<128, 8, 1>(qq, kk, vv, o, lse, o_prev, lse_prev, Nq, Nkv, H, Bq, P, scale_log2, n_qtiles, work, out_f32, stream);
    else if (D == 128 && keysplit)
        launch_schedule<128, 8, 2>(qq, kk, vv, o, lse, o_prev, lse_prev, Nq, Nkv, H, Bq, P, scale_log2, n_qtiles, work, out_f32, stream);
    else if (D == 128)
        launch_schedule<128, 4, 1>(qq, kk, vv, o, lse, o_prev, lse_prev, Nq, Nkv, H, Bq, P, scale_log2, n_qtiles, work, out_f32, stream);
    else
        launch_schedule<64, 4, 1>(qq, kk, vv, o, lse, o_prev, lse_prev, Nq, Nkv, H, Bq, P, scale_log2, n_qtiles, work, out_f32, stream);
    e = hipGetLastError();
    if (ws != nullptr) {
        const hipError_t f = hipFreeAsync(ws, stream);   // stream-ordered: after the kernel
        if (e == hipSuccess) e = f;
    }
    return e;
}

}  // namespace dtl
