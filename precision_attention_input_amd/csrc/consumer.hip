// consumer.hip -- attention over one destination's unpacked tensors (gfx950 MFMA).
//
// A check of the unpacked layouts from the consumer's side, not a step of the pack/unpack
// path: the unpack_for_sage page hands q8, k8 (INT8 [B, S, h, D], one FP32 scale per
// 64-row group in q_scale / k_scale [B, h, W]) and v8 (FP8 E4M3 [B, D, h, Spad]) to a Sage
// attention kernel, the V scale staying with the caller (Returns).  This kernel reads them
// that way over the live rows t < used:
//   score(i, t) = (q8[i] . k8[t]) * q_scale[i / 64] * k_scale[t / 64] / sqrt(D)
//   out[i, d]   = sum_t softmax_t(score(i, .)) * e4m3(v8[d, t]) * v_scale[d]
// with the INT8 dot products on gfx950's v_mfma_i32_16x16x64_i8 (exact int32) and the P.V
// product on v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit block scales), P
// quantized to E4M3 after scaling by 448 (the largest E4M3 value), as an FP8 consumer does.  Smooth K needs no correction: removing a per-channel
// mean from every key shifts all scores of a query by the same amount.
//
// Work decomposition: a 256-thread workgroup owns 64 query rows of one (b, head) -- one Q
// scale group -- and each wave 16 of them.  Key tiles of 128 rows (two K scale groups) and
// the matching 128 columns of v8 are copied with coalesced 16-byte loads into
// double-buffered LDS tiles shared by the four waves; the next tile's loads are in flight
// while the current one is computed.  Both products are computed transposed, so that every
// per-query quantity lives in the lanes of that query's column:
//   S^T[key, q] = K . Q^T   (A = 16 keys x 64 channels of k8, B = 64 channels x 16 queries)
//   O^T[d, q]  += V^T . P^T (A = 16 channels x 128 keys of v8, B = 128 keys x 16 queries)
// Lane l of an MFMA operand holds row / column l % 16 and the bytes of lane group l / 16;
// both instructions pair byte i of lane group g of A with byte i of lane group g of B
// (checked on gfx950 with an in-bounds one-hot probe), so any assignment of the reduced
// index to (lane group, byte), the same for both operands, gives the full sum.  The
// accumulator lane l holds rows 4 * (l / 16) + [0, 4) of column l % 16.  The rows of the
// K operand are fed in a permuted order -- row i of 16-key block kb is key
// 32 (i / 4) + 4 kb + i % 4 -- so the accumulators of lane group g hold the 32 consecutive
// keys 32 g + [0, 32) (byte 4 kb + r = key 32 g + 4 kb + r): the lane's packed P bytes are
// then the P.V product's B operand in key order, the V^T fragment is 32 consecutive bytes
// of a channel row, and each lane's keys share one K scale group.  No data moves between
// lanes except the max / sum reductions over the four lanes of a query.  The permutation is
// applied once, when a K row is stored in LDS (slot 16 kb + 4 q + r for key 32 q + 4 kb + r),
// so every fragment read covers 16 consecutive padded rows.
#include <cmath>

#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kConsumerKeys = 128;   // keys per LDS tile: one P.V MFMA per channel block
// Waves (16 queries each) per workgroup: they share every K / V tile in LDS, so more waves
// mean fewer tile loads per query; 8 measured best at D = 128, 4 at D = 64.
template <int D>
constexpr int consumer_waves() { return D == 128 ? 8 : 4; }
constexpr int kUnitScale = 127;      // E8M0 block scale 2^0
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)

struct ConsumerParams {
    const int8_t *q8, *k8;
    const uint8_t* v8;
    const float *q_scale, *k_scale, *v_scale;
    float* out;
    int64_t S, h, spad, W, used;
    float score_scale;   // log2(e) / sqrt(D)
};


// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query's lanes), left in all
// four, with gfx950's lane-swap instructions: v_permlane16_swap exchanges rows 1 and 3 of one
// register with rows 0 and 2 of another, v_permlane32_swap the upper half of one with the
// lower half of another; both operands are copies of v, so each result lane meets its
// partner's value.  No LDS traffic.  The sum is (r0 + r1) + (r2 + r3) in every lane.
__device__ __forceinline__ float quad_max(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(v);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(v);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS tiles: KT keys x D channels of k8 and D channels x KT keys of v8, rows padded by 16
// bytes (keeps 16-byte writes aligned and spreads the fragment reads over the banks).
template <int D, int KT>
struct ConsumerTiles {
    static constexpr int KROW = D + 16, VROW = KT + 16;
    static constexpr int KBYTES = KT * KROW, VBYTES = D * VROW;
    uint8_t k[2][KBYTES];
    uint8_t v[2][VBYTES];
};

template <int D>
__global__ __launch_bounds__(64 * consumer_waves<D>()) __attribute__((amdgpu_waves_per_eu(2)))
void consumer_kernel(
    ConsumerParams p) {
    constexpr int KT = kConsumerKeys;          // keys per tile
    constexpr int KB = KT / 16;                // 16-key blocks of S^T per tile
    constexpr int KC = D / 64;                 // 64-channel slices of a Q / K row
    constexpr int CB = D / 16;                 // 16-channel blocks of the output
    using T = ConsumerTiles<D, KT>;
    // global -> LDS copy of one tile: 16 bytes per thread per step
    constexpr int KV = D / 16;                 // 16-byte pieces of a K row
    constexpr int VV = KT / 16;                // 16-byte pieces of a V row
    constexpr int NT = 64 * consumer_waves<D>();   // threads per workgroup
    constexpr int NQ = 16 * consumer_waves<D>();   // queries per workgroup
    constexpr int KSTEPS = KT * KV / NT;
    constexpr int VSTEPS = D * VV / NT;
    static_assert(KSTEPS * NT == KT * KV && VSTEPS * NT == D * VV, "tile split");
    __shared__ __align__(16) T tl;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int64_t hD = p.h * D;
    const int64_t qi = tile * NQ + wave * 16 + col;   // this lane's query

    // Q^T fragments (B operand): channels 64c + 16 grp + [0, 16) of query qi.
    v4i qf[KC];
    const int8_t* qrow = p.q8 + (b * p.S + qi) * hD + j * D + 16 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c)
        qf[c] = qi < p.S ? *reinterpret_cast<const v4i*>(qrow + 64 * c) : v4i{0, 0, 0, 0};
    // Q scale group of this wave's queries; a wave wholly past `used` (it still takes part
    // in the shared tile loads and barriers, its outputs are not stored) reads the last one.
    const int64_t qg = min((tile * NQ + wave * 16) / 64, p.W - 1);
    const float qs = p.q_scale[(b * p.h + j) * p.W + qg] * p.score_scale;
    const float* ksc = p.k_scale + (b * p.h + j) * p.W;

    v4f o[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -__builtin_inff(), lsum = 0.0f;

    const int64_t ntiles = (p.used + KT - 1) / KT;
    const int8_t* kg = p.k8 + b * p.S * hD + j * D;
    const uint8_t* vg = p.v8 + ((b * D) * p.h + j) * p.spad;
    const int64_t vrow = p.h * p.spad;         // bytes between channel rows of v8

    // Coalesced tile loads into registers (rows of k8 are 16-byte pieces of D bytes; rows
    // of the tile's v8 are KT bytes of one channel).  K rows past `used` and V columns past
    // Spad are zero.
    uint4 kr[KSTEPS], vr[VSTEPS];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const int e = s * NT + tid, row = e / KV, piece = e % KV;
            const int64_t t = t0 + row;
            kr[s] = t < p.used ? *reinterpret_cast<const uint4*>(kg + t * hD + 16 * piece)
                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < VSTEPS; ++s) {
            const int e = s * NT + tid, d = e / VV, piece = e % VV;
            const int64_t t = t0 + 16 * piece;
            vr[s] = t < p.spad ? *reinterpret_cast<const uint4*>(vg + d * vrow + t)
                               : make_uint4(0, 0, 0, 0);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const int e = s * NT + tid, row = e / KV, piece = e % KV;
            const int slot = 16 * ((row & 31) >> 2) + 4 * (row >> 5) + (row & 3);
            *reinterpret_cast<uint4*>(&tl.k[buf][slot * T::KROW + 16 * piece]) = kr[s];
        }
#pragma unroll
        for (int s = 0; s < VSTEPS; ++s) {
            const int e = s * NT + tid, d = e / VV, piece = e % VV;
            *reinterpret_cast<uint4*>(&tl.v[buf][d * T::VROW + 16 * piece]) = vr[s];
        }
    };
    fetch(0);
    stash(0);
    __syncthreads();

    for (int64_t kt = 0; kt < ntiles; ++kt) {
        const int buf = (int)(kt & 1);
        const int64_t t0 = kt * KT;
        if (kt + 1 < ntiles) fetch(t0 + KT);   // in flight while this tile is computed
        const uint8_t* kl = tl.k[buf];
        const uint8_t* vl = tl.v[buf];
        // S^T, 16 keys per MFMA: row i of block kb is key 32 (i / 4) + 4 kb + i % 4 of the
        // tile, so the accumulator rows 4 grp + r of every block hold this lane's 32
        // consecutive keys 32 grp + 4 kb + r.
        // (The stash stores key row 32 q + 4 kb + r in LDS slot 16 kb + 4 q + r, so block
        // kb reads 16 consecutive slots: no bank conflicts.)
        v4i s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = v4i{0, 0, 0, 0};
            const uint8_t* krow = kl + (16 * kb + col) * T::KROW + 16 * grp;
#pragma unroll
            for (int c = 0; c < KC; ++c)
                s[kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    *reinterpret_cast<const v4i*>(krow + 64 * c), qf[c], s[kb], 0, 0, 0);
        }
        // The lane's keys lie in one 64-key K scale group (positive; a group past the scale
        // width holds no live key and takes 1), so its largest score is its largest dot
        // product times that scale.  The int32 dot products convert exactly; only the last
        // tile can hold keys past `used`, which become -inf (no maximum, probability 0).
        const int live = (int)min((int64_t)KT, p.used - t0);   // live keys of this tile
        const int64_t gi = t0 / 64 + (grp >> 1);
        const float scl = gi < p.W ? qs * ksc[gi] : 1.0f;
        float xf[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) xf[kb][r] = (float)s[kb][r];
        if (live < KT) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (32 * grp + 4 * kb + r >= live) xf[kb][r] = -__builtin_inff();
        }
        float gmax = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) gmax = fmaxf(gmax, xf[kb][r]);
        float tmax = gmax * scl;
        tmax = quad_max(tmax);
        const float mnew = fmaxf(m, tmax);           // finite: key t0 < used is live
        // 448 p = exp2(score - mnew + log2(448)), one fma and one exp2 per key; the row sum
        // is kept in the same 448-scaled units.  The values stay at or below 448 (up to the
        // exp2 error), so the E4M3 conversion needs no clamp.
        const float moff = mnew - kLog2_448;
        float psum = 0.0f;
        uint32_t pw[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(xf[kb][r], scl, -moff));
                psum += pr[r];
            }
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
            pw[kb] = (uint32_t)w;
        }
        psum = quad_sum(psum);
        // Rescale the running sums only when some query's maximum moved in this wave.
        if (__builtin_amdgcn_ballot_w64(mnew != m) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            lsum *= alpha;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;
        }
        lsum += psum;
        m = mnew;
        // P^T fragment: the lane's 32 keys, byte 4 kb + r = key 32 grp + 4 kb + r, i.e. in
        // key order; the V^T rows (channels) supply the same 32 consecutive keys.
        const v8i pf = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                        (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint4* v16 =
                reinterpret_cast<const uint4*>(vl + (16 * cb + col) * T::VROW + 32 * grp);
            const uint4 va0 = v16[0], va1 = v16[1];
            const v8i va = {(int)va0.x, (int)va0.y, (int)va0.z, (int)va0.w,
                            (int)va1.x, (int)va1.y, (int)va1.z, (int)va1.w};
            o[cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                va, pf, o[cb], 0, 0, 0, kUnitScale, 0, kUnitScale);
        }
        if (kt + 1 < ntiles) stash(buf ^ 1);   // the other buffer: nobody reads it now
        __syncthreads();
    }

    if (qi >= p.used) return;
    const float inv = 1.0f / lsum;                 // lsum is in 448-scaled units
    float* orow = p.out + (b * p.used + qi) * hD + j * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int d0 = cb * 16 + 4 * grp;
        float4 r = make_float4(o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv);
        if (p.v_scale) {
            const float4 vs =
                *reinterpret_cast<const float4*>(p.v_scale + (b * p.h + j) * D + d0);
            r.x *= vs.x;
            r.y *= vs.y;
            r.z *= vs.z;
            r.w *= vs.w;
        }
        *reinterpret_cast<float4*>(orow + d0) = r;
    }
}

}  // namespace

hipError_t launch_consumer(const ConsumerLaunch& a, hipStream_t stream) {
    ConsumerParams p;
    p.q8 = a.q8;
    p.k8 = a.k8;
    p.v8 = a.v8;
    p.q_scale = a.q_scale;
    p.k_scale = a.k_scale;
    p.v_scale = a.v_scale;
    p.out = a.out;
    p.S = a.S;
    p.h = a.h;
    p.spad = (a.S + kGroup - 1) / kGroup * kGroup;
    p.W = a.W;
    p.used = a.used;
    p.score_scale = (float)(1.4426950408889634 / std::sqrt((double)a.D));
    if (a.D == 64) {
        constexpr int nq = 16 * consumer_waves<64>();
        const dim3 grid((unsigned)((a.used + nq - 1) / nq), (unsigned)a.h, (unsigned)a.B);
        hipLaunchKernelGGL((consumer_kernel<64>), grid, dim3(4 * nq), 0, stream, p);
    } else {
        constexpr int nq = 16 * consumer_waves<128>();
        const dim3 grid((unsigned)((a.used + nq - 1) / nq), (unsigned)a.h, (unsigned)a.B);
        hipLaunchKernelGGL((consumer_kernel<128>), grid, dim3(4 * nq), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace ulp
