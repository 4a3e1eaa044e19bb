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
// quantized to E4M3 after scaling by 448 (the largest E4M3 value), as an FP8 consumer does.
// Each row is normalized by the sum of its rounded probabilities, formed on the matrix
// cores in the same products as the output (a Sage consumer sums the unrounded ones in
// FP32; either is a valid normalization of the rounded weights).
// Smooth K needs no correction: removing a per-channel mean from every key shifts all scores
// of a query by the same amount.
//
// Work decomposition: a workgroup of WAVES waves owns WAVES x QB x 16 query rows of one
// (b, head); a wave owns QB column blocks of 16 queries, all in one Q scale group.  Key
// tiles of 128 rows (two K scale groups) and the matching 128 columns of v8 are loaded from
// memory straight into double-buffered LDS tiles shared by the waves; the next tile's loads
// are in flight while the current one is computed.  Both products are computed transposed,
// so that every per-query quantity lives in the lanes of that query's column:
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
// lanes except the max reduction over the four lanes of a query.  The permutation is
// applied once, when a K row lands in LDS (slot 16 kb + 4 q + r for key 32 q + 4 kb + r),
// so every fragment read covers 16 consecutive rows.
#include <cmath>
#include <type_traits>

#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kConsumerKeys = 128;   // keys per LDS tile: one P.V MFMA per channel block
// Workgroup shape: WAVES waves of QB 16-query column blocks each.  The QB blocks of a wave
// share every K / V fragment read from LDS (one fragment feeds QB MFMAs), so LDS traffic
// per FLOP falls as 1 / QB; the waves of a workgroup share every tile loaded into LDS.
// The launcher picks the shape (see launch_consumer).
constexpr int kUnitScale = 127;      // E8M0 block scale 2^0
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)
// The S^T accumulators start at the bit pattern of 1.5 * 2^23 instead of 0.  Binary32
// values in [2^23, 2^24) are the integers, one per bit pattern, so for any dot product d
// with |d| < 2^22 (127 * 127 * D <= 2064512 here) the accumulator's bits read as a float
// are exactly 1.5 * 2^23 + d: the scores need no integer-to-float conversion.
constexpr int kDotBias = 0x4B400000;
constexpr float kDotBiasF = 12582912.0f;
constexpr int kE4M3One = 0x38;       // E4M3 encoding of 1.0

struct ConsumerParams {
    const int8_t *q8, *k8;
    const uint8_t* v8;
    const float *q_scale, *k_scale, *v_scale;
    float* out;
    int64_t S, h, spad, W, used;
    float score_scale;   // log2(e) / sqrt(D)
};


// Max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query's lanes), left in all four,
// with gfx950's lane-swap instructions: v_permlane16_swap exchanges rows 1 and 3 of one
// register with rows 0 and 2 of another, v_permlane32_swap the upper half of one with the
// lower half of another; both operands are copies of v, so each result lane meets its
// partner's value.  No LDS traffic.
__device__ __forceinline__ float quad_max(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(v);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS tiles: KT key slots x D channels of k8 and D channels x KT keys of v8, unpadded.  The
// 16-byte pieces of each row are stored XOR-permuted by the row index (the piece swizzle
// below), so the 16 rows x 16 bytes of a fragment read fall in distinct banks.
template <int D, int KT>
struct ConsumerTiles {
    static constexpr int KBYTES = KT * D, VBYTES = D * KT;
    uint8_t k[2][KBYTES];
    uint8_t v[2][VBYTES];
};

// Stored position of 16-byte piece `lp` of K slot `slot` (rows of D bytes: two slots share
// a 128-byte line at D = 64) and of V row `row` (rows of 128 bytes).  Each is its own
// inverse, so the same function maps a stored position back to the piece.
template <int D>
__device__ __forceinline__ int k_piece(int slot, int lp) {
    return D == 128 ? lp ^ (slot & 7) : lp ^ ((slot >> 1) & 3);
}
__device__ __forceinline__ int v_piece(int row, int lp) { return lp ^ (row & 7); }

// Buffer resource for raw buffer loads: 64-bit base, stride 0, `bytes` in range (loads at
// or past it return zeros), default data format.
__device__ __forceinline__ v4i buffer_resource(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return v4i{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// Global -> LDS buffer load of 16 bytes per lane: lane l's bytes land at LDS address
// lds + 16 l (`lds` is the wave's, in M0; the hardware adds the lane offset).  Written as
// asm so that the compiler, which cannot tell the two LDS tile buffers apart, does not wait
// for these loads before every later LDS read: the loads into one buffer overlap the reads
// of the other, and lds_load_barrier() waits for them explicitly.  The asm writes no
// register the compiler sees (the data goes to LDS); M0 is used by nothing else here.
__device__ __forceinline__ void buffer_load_lds16(v4i rsrc, uint32_t lds, int voffset) {
    // rsrc and lds are uniform; readfirstlane makes the compiler hold them in SGPRs
    const v4i rs = {__builtin_amdgcn_readfirstlane(rsrc[0]),
                    __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]),
                    __builtin_amdgcn_readfirstlane(rsrc[3])};
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rs) : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Wait for all of this wave's outstanding memory operations (the LDS loads included), then
// for every wave of the workgroup.  The wait is the compiler's own instruction, so it knows
// that every earlier load has completed and adds no waits of its own after it (a compiler
// wait would count the LDS loads it does not see and drain them).
__device__ __forceinline__ void lds_load_barrier() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

template <int D, int QB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void consumer_kernel(ConsumerParams p) {
    constexpr int KT = kConsumerKeys;          // keys per tile
    constexpr int KB = KT / 16;                // 16-key blocks of S^T per tile
    constexpr int KC = D / 64;                 // 64-channel slices of a Q / K row
    constexpr int CB = D / 16;                 // 16-channel blocks of the output
    using T = ConsumerTiles<D, KT>;
    constexpr int NQW = 16 * QB;               // queries per wave
    constexpr int NQ = NQW * WAVES;            // queries per workgroup
    static_assert(64 % NQW == 0, "a wave's queries share one Q scale group");
    static_assert(127 * 127 * D < (1 << 22), "biased dot products stay in [2^23, 2^24)");
    // global -> LDS copy of one tile pair in 1 KB pieces, one wave instruction each
    constexpr int NKC = KT * D / 1024, NVC = D * KT / 1024;
    constexpr int CPW = (NKC + NVC) / WAVES;   // pieces per wave
    static_assert(CPW * WAVES == NKC + NVC, "tile split");
    __shared__ __align__(16) T tl;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS load bases
    const int col = lane & 15, grp = lane >> 4;
    const int64_t tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int64_t hD = p.h * D;
    const int64_t qw = tile * NQ + wave * NQW;   // first query of this wave
    // this lane's query in column block qb: qw + 16 qb + col

    // Q^T fragments (B operand): channels 64c + 16 grp + [0, 16) of each of the lane's queries.
    v4i qf[QB][KC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qi = qw + 16 * qb + col;
        const int8_t* qrow = p.q8 + (b * p.S + qi) * hD + j * D + 16 * grp;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            qf[qb][c] = qi < p.S ? *reinterpret_cast<const v4i*>(qrow + 64 * c)
                                 : v4i{0, 0, 0, 0};
    }
    // Q scale group of this wave's queries; a wave wholly past `used` (it still takes part
    // in the shared tile loads and barriers, its outputs are not stored) reads the last one.
    const int64_t qg = min(qw / 64, p.W - 1);
    const float qs = p.q_scale[(b * p.h + j) * p.W + qg] * p.score_scale;
    const float* ksc = p.k_scale + (b * p.h + j) * p.W;

    // o: the output sums O^T; ls: the row sums, one more O^T block whose 16 "channels" are
    // all E4M3 ones, so every element of ls[qb] is the sum of the rounded probabilities of
    // the lane's query; m: the running maximum (log2 units).
    v4f o[QB][CB], ls[QB];
    float m[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[qb][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        ls[qb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        m[qb] = -__builtin_inff();
    }

    const int64_t ntiles = (p.used + KT - 1) / KT;
    const int8_t* kg = p.k8 + b * p.S * hD + j * D;
    const uint8_t* vg = p.v8 + ((b * D) * p.h + j) * p.spad;
    const int64_t vrow = p.h * p.spad;         // bytes between channel rows of v8

    // Tile loads straight into LDS.  Piece c of the pair is K (c < NKC) or V; lane l of
    // its instruction fills stored bytes 1024 c' + 16 l, i.e. a (row, stored piece), and
    // loads the global bytes of the logical piece stored there.  K rows past `used` lie at
    // or past the K range and read as zeros; V columns past Spad are pointed past the V
    // range (0x80000000) and read as zeros; the ranges end inside batch entry b.
    const uint32_t vbytes_b = (uint32_t)(D * vrow - j * p.spad);   // vg .. end of entry b
    // The lane's part of each of the wave's CPW pieces, the same for every tile: the byte
    // offset it loads from, relative to the tile's first key (K) or column (V), and for V
    // the tile column it starts at.
    int ld_off[CPW], ld_col[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave + WAVES * i;
        if (c < NKC) {
            const int off = c * 1024 + 16 * lane;
            const int slot = off / D, lp = k_piece<D>(slot, (off % D) / 16);
            // LDS slot 16 kb + 4 q + r holds key 32 q + 4 kb + r of the tile
            const int key = 32 * ((slot & 15) >> 2) + 4 * (slot >> 4) + (slot & 3);
            ld_off[i] = key * (int)hD + 16 * lp;
            ld_col[i] = 0;
        } else {
            const int off = (c - NKC) * 1024 + 16 * lane;
            const int row = off / KT, lp = v_piece(row, (off % KT) / 16);
            ld_off[i] = row * (int)vrow + 16 * lp;
            ld_col[i] = 16 * lp;
        }
    }
    const uint32_t lds_k = lds_address(tl.k[0]), lds_v = lds_address(tl.v[0]);
    // Loads of the K tile of keys [tk, tk + KT) into K buffer kbuf and of the V tile of
    // keys [tv, tv + KT) into V buffer vbuf, each only if asked for (k_on / v_on are
    // uniform).
    auto issue = [&](int kbuf, int64_t tk, bool k_on, int vbuf, int64_t tv, bool v_on) {
        const v4i krs = buffer_resource(kg + tk * hD, (uint32_t)((p.used - tk) * hD));
        const v4i vrs = buffer_resource(vg + tv, vbytes_b - (uint32_t)tv);
        const int vlive = (int)min((int64_t)KT, p.spad - tv);   // columns before Spad
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = wave + WAVES * i;
            if (c < NKC) {
                if (k_on)
                    buffer_load_lds16(krs, lds_k + kbuf * T::KBYTES + c * 1024, ld_off[i]);
            } else if (v_on) {
                buffer_load_lds16(vrs, lds_v + vbuf * T::VBYTES + (c - NKC) * 1024,
                                  ld_col[i] < vlive ? ld_off[i] : (int)0x80000000);
            }
        }
    };
    // K scale of the lane's 64-key group in the tile starting at t0 (positive; a group past
    // the scale width holds no live key and takes 1), loaded a tile ahead so that it is in
    // a register when the tile's barrier has passed.
    auto k_scale_of = [&](int64_t t0) {
        const int64_t gi = t0 / 64 + (grp >> 1);
        return gi < p.W ? ksc[gi] : 1.0f;
    };

    // S^T of one tile from its K tile kl, 16 keys per MFMA: row i of block kb is key
    // 32 (i / 4) + 4 kb + i % 4 of the tile, so the accumulator rows 4 grp + r of every
    // block hold this lane's 32 consecutive keys 32 grp + 4 kb + r.  (The loads store key
    // row 32 q + 4 kb + r in LDS slot 16 kb + 4 q + r, so block kb reads 16 consecutive
    // slots.)  Each K fragment read from LDS feeds the MFMAs of all QB column blocks.  The
    // sums start from kDotBias.
    auto s_tile = [&](const uint8_t* kl, v4i (&s)[QB][KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[qb][kb] = v4i{kDotBias, kDotBias, kDotBias, kDotBias};
            const int slot = 16 * kb + col;
            const uint8_t* krow = kl + slot * D;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const v4i kf = *reinterpret_cast<const v4i*>(
                    krow + 16 * k_piece<D>(slot, grp + 4 * c));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qf[qb][c], s[qb][kb],
                                                                       0, 0, 0);
            }
        }
    };

    // Softmax of the tile starting at t0 from its biased dot products s: the running maximum
    // moves on, pw gets the packed E4M3 probabilities (scaled by 448), and alpha / resc say
    // how the output and row sums must be rescaled before the tile's P.V is added (resc is
    // false, uniformly over the wave, when no query's maximum moved).  `last` (a
    // compile-time tag) marks the final tile, the only one that can hold keys past `used`;
    // the other tiles carry no masking code.
    auto softmax = [&](auto last, v4i (&s)[QB][KB], int64_t t0, float ks,
                       uint32_t (&pw)[QB][KB], float (&alpha)[QB], bool (&resc)[QB]) {
        // The lane's keys lie in one 64-key K scale group, so its largest score is its
        // largest dot product times that scale.  xf = 1.5 * 2^23 + dot exactly (kDotBias),
        // ordered as the dot products are; only the last tile can hold keys past `used`,
        // which become -inf (no maximum, probability 0).
        // key 32 grp + i of the tile is live iff i < lim (compared against the constant i)
        const int lim = (int)min((int64_t)KT, p.used - t0) - 32 * grp;
        const float scl = t0 / 64 + (grp >> 1) < p.W ? qs * ks : 1.0f;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float xf[KB][4];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) xf[kb][r] = __int_as_float(s[qb][kb][r]);
            if constexpr (decltype(last)::value) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * kb + r >= lim) xf[kb][r] = -__builtin_inff();
            }
            float gmax = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) gmax = fmaxf(gmax, xf[kb][r]);
            float tmax = (gmax - kDotBiasF) * scl;   // the subtraction is exact
            tmax = quad_max(tmax);
            const float mnew = fmaxf(m[qb], tmax);   // finite: key t0 < used is live
            // 448 p = exp2(score - mnew + log2(448)) = exp2(xf * scl - moff), one fma and one
            // exp2 per key, with the bias folded into moff (rounded once: the exponent of
            // every key of the lane is off by at most half an ulp of moff, about
            // 2^-24 * 1.5 * 2^23 * scl).  The values stay at or below 448 (up to that and
            // the exp2 error), so the E4M3 conversion needs no clamp.
            const float moff = __builtin_fmaf(kDotBiasF, scl, mnew - kLog2_448);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float pr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(xf[kb][r], scl, -moff));
                // the first conversion writes the low half and keeps the high half of its
                // last operand, which the second overwrites: any bits do (an empty asm
                // defines them without an instruction; a constant would cost a move)
                int w;
                asm volatile("" : "=v"(w));
                w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], w, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
                pw[qb][kb] = (uint32_t)w;
            }
            // Rescale the running sums only when some query's maximum moved in this wave.
            resc[qb] = __builtin_amdgcn_ballot_w64(mnew != m[qb]) != 0;
            alpha[qb] = resc[qb] ? __builtin_amdgcn_exp2f(m[qb] - mnew) : 1.0f;
            m[qb] = mnew;
        }
    };
    auto rescale = [&](const float (&alpha)[QB], const bool (&resc)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            if (resc[qb]) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) o[qb][cb] *= alpha[qb];
                ls[qb] *= alpha[qb];
            }
    };

    // O^T += V^T P^T for one tile from its V tile vl.  P^T fragment: the lane's 32 keys,
    // byte 4 kb + r = key 32 grp + 4 kb + r, i.e. in key order; the V^T rows (channels)
    // supply the same 32 consecutive keys.  Each V fragment read from LDS feeds the MFMAs
    // of all QB column blocks.  One more MFMA per column block, with an A operand of E4M3
    // ones, adds the rounded probabilities of each query to its row sum.
    auto pv_tile = [&](const uint8_t* vl, const uint32_t (&pw)[QB][KB]) {
        v8i pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            pf[qb] = v8i{(int)pw[qb][0], (int)pw[qb][1], (int)pw[qb][2], (int)pw[qb][3],
                         (int)pw[qb][4], (int)pw[qb][5], (int)pw[qb][6], (int)pw[qb][7]};
        v8i vas[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int row = 16 * cb + col;
            const uint8_t* vr = vl + row * KT;
            const uint4 va0 = *reinterpret_cast<const uint4*>(vr + 16 * v_piece(row, 2 * grp));
            const uint4 va1 =
                *reinterpret_cast<const uint4*>(vr + 16 * v_piece(row, 2 * grp + 1));
            vas[cb] = v8i{(int)va0.x, (int)va0.y, (int)va0.z, (int)va0.w,
                          (int)va1.x, (int)va1.y, (int)va1.z, (int)va1.w};
        }
        // with eight waves, all of the tile's V fragment reads are issued before its first
        // P.V product (measured: 1-2 % faster); the smaller shapes leave the order to the
        // compiler
        if constexpr (WAVES == 8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const v8i va = vas[cb];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                o[qb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    va, pf[qb], o[qb][cb], 0, 0, 0, kUnitScale, 0, kUnitScale);
        }
        constexpr int ones4 = kE4M3One * 0x01010101;
        const v8i ones = {ones4, ones4, ones4, ones4, ones4, ones4, ones4, ones4};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            ls[qb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                ones, pf[qb], ls[qb], 0, 0, 0, kUnitScale, 0, kUnitScale);
    };

    // Tile by tile: the next tile's loads (into the other buffer) are in flight while this
    // tile's products and softmax run; they complete by the barrier after it.
    float ks_next = k_scale_of(0);
    issue(0, 0, true, 0, 0, true);
    lds_load_barrier();
    auto step = [&](auto last, int buf, int64_t t0, bool next) {
        const float ks = ks_next;
        if (next) {
            ks_next = k_scale_of(t0 + KT);
            issue(buf ^ 1, t0 + KT, true, buf ^ 1, t0 + KT, true);
        }
        v4i s[QB][KB];
        s_tile(tl.k[buf], s);
        uint32_t pw[QB][KB];
        float alpha[QB];
        bool resc[QB];
        softmax(last, s, t0, ks, pw, alpha, resc);
        rescale(alpha, resc);
        pv_tile(tl.v[buf], pw);
    };
    for (int64_t kt = 0; kt + 1 < ntiles; ++kt) {
        step(std::false_type{}, (int)(kt & 1), kt * KT, true);
        lds_load_barrier();   // the next pair has landed; this one is no longer read
    }
    step(std::true_type{}, (int)((ntiles - 1) & 1), (ntiles - 1) * KT, false);
    // The last tile's results are used only by the lanes of live queries (the branch
    // below).  MFMAs need every lane of the wave, so they must not run inside that branch:
    // an opaque use of every accumulator here, where all lanes are active, keeps the
    // compiler from moving the last tile's MFMAs (or anything feeding them) into it.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) asm volatile("" : "+v"(o[qb][cb]));
        asm volatile("" : "+v"(ls[qb]));
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qi = qw + 16 * qb + col;
        if (qi >= p.used) continue;
        const float inv = 1.0f / ls[qb][0];        // the row sum, in 448-scaled units
        float* orow = p.out + (b * p.used + qi) * hD + j * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int d0 = cb * 16 + 4 * grp;
            float4 r = make_float4(o[qb][cb][0] * inv, o[qb][cb][1] * inv,
                                   o[qb][cb][2] * inv, o[qb][cb][3] * inv);
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
}

template <int D, int QB, int WAVES>
void launch_shape(const ConsumerLaunch& a, const ConsumerParams& p, hipStream_t stream) {
    constexpr int nq = 16 * QB * WAVES;   // queries per workgroup
    const dim3 grid((unsigned)((a.used + nq - 1) / nq), (unsigned)a.h, (unsigned)a.B);
    hipLaunchKernelGGL((consumer_kernel<D, QB, WAVES>), grid, dim3(64 * WAVES), 0, stream, p);
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
    // Shapes, measured: at D = 128, 8 waves x 2 column blocks (256 queries per workgroup,
    // one workgroup per CU) when that still gives at least two workgroups per CU of the
    // 256, else 4 waves x 1 block (64 queries, several workgroups per CU); at D = 64, 4 x 1.
    if (a.D == 64) {
        launch_shape<64, 1, 4>(a, p, stream);
    } else if ((a.used + 255) / 256 * a.h * a.B >= 512) {
        launch_shape<128, 2, 8>(a, p, stream);
    } else {
        launch_shape<128, 1, 4>(a, p, stream);
    }
    return hipGetLastError();
}

}  // namespace ulp
