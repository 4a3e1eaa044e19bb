// stats_pack.hip -- statistics and pack of the shards from one read of Q, K and V (gfx950).
//
// As the pages lay the step out, Q and K are read twice: once by k_grouped_amax (with the
// boundary min/max that derive_k_boundary_amax consumes), once more by the pack that uses
// the resulting per-group scales (k_grouped_amax page, description).  Yet derive can change
// only two slots of a rank, its first and last, and of those only a slot whose group
// another rank also touches, or whose rows all lie in the zero tail (its min/max is then
// empty and derive leaves the floor, while the grouped amax ran over the zero rows).  Every
// other slot's amax is final once this rank has seen the group's rows.
//
// Phase 0: one 256-thread workgroup per (rank, b, slot, tensor, 256 channels: two heads at
// D = 128, four at D = 64) loads the rank's rows of the group (at most 64, eight per
// thread) of its tensor once.  A Q or K workgroup reduces the raw |Q| or centered
// |K - mean| amax of each head (and, for the first and last slot, the per-channel raw
// min/max) in the same registers, writes them, and quantizes the rows with the new scales,
// unless the slot must wait for derive; a V workgroup, which needs no statistic, converts
// its rows to E4M3.  One tensor per workgroup makes each row access a 512-byte run (Q and K
// together in one workgroup would read two 256-byte runs per row: measured 5 % slower on
// the same bytes).  Phase 1, after the min/max are gathered: one workgroup per (rank, b,
// first or last slot, 128 channels) derives the slot's amax for Q and K as
// derive_k_boundary_amax (description) does, writes it, and, if the slot waited, re-reads
// its rows and quantizes them with it.  The outputs are bit-identical to the separate
// statistics, derive and pack launches: the same amax (a direct max of the same
// |RN(x - mean)| values, which the min/max identity of derive_k_boundary_amax equals
// exactly), the same chunk bytes.
#include "pack_device.h"
#include "ulp_kernels.h"


namespace ulp {
namespace {


struct StatsPackParams {
    const uint16_t *q, *k, *v, *mean;
    const float* v_scale;
    float *q_amax, *k_amax, *q_minmax, *k_minmax;
    uint8_t* send;
    int64_t dest_stride, x_rank_stride, amax_rank_stride, minmax_rank_stride, send_rank_stride;
    int64_t gathered_stride;    // phase 1: floats between ranks of the gathered min/max
    int64_t B, L, H, h, P, S, used, slots, sec, ssec;
    int rank0;
    int nhb;          // channel blocks per row: of 256 channels (phase 0), 128 (phase 1)
    int grid_slots;   // slots per (rank, b) in the grid: every slot (phase 0), 2 (phase 1)
};

// Whether slot j of a rank with n touched slots must be quantized after derive (above).
__device__ __forceinline__ bool waits_for_derive(int64_t rank, int64_t L, int64_t S,
                                                 int64_t used, int64_t j, int64_t n) {
    if (j != 0 && j != n - 1) return false;
    const int64_t g = first_group(rank, L) + j;
    const int64_t lo = max(kGroup * g, rank * L), hi = min(kGroup * g + kGroup, rank * L + L);
    const bool shared = kGroup * g < rank * L || min(kGroup * g + kGroup, S) > hi;
    return shared || min(hi, used) <= lo;
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 8-byte global store (NT: non-temporal).
template <bool NT>
__device__ __forceinline__ void store8(void* p, uint32_t lo, uint32_t hi) {
    if constexpr (NT) {
        const u32x2_t w = {lo, hi};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
    } else {
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    }
}

// The rows of one group (at most 64) and 256 channels of one tensor, as the threads of a
// phase-0 workgroup hold them: lane bits 0-4 pick a 16-byte piece (8 channels) of the
// workgroup's 512-byte run of a row, the row lane rq = 2 * wave + lane bit 5 picks rows
// rq + 8 i, i < 8.  The lanes of one head differ in the piece bits inside the head (0-3 at
// D = 128, 0-2 at D = 64) and in bit 5.
struct Tile {
    int64_t b, j, g, n, lo, hi, l0;
    int nrow, namax;
    int cq, rq, hib, pc;    // piece, row lane, head lane group in the block, piece in the head
    bool valid;             // the piece lies inside the row (a ragged last block has 128)
    int64_t head;           // global head of the piece (of the piece read, if !valid)
};

// LDS of a phase-0 workgroup: the per-wave head maxima and the [row lane][channel] min/max
// table (both Q and K tiles use the same arrays).
struct Phase0Lds {
    float red[4][256 / 64];
    float col[8][256 + 1];
};

// Stats, scale and codes of one Q (CENTER false) or K (CENTER true) tile.
template <int DT, int D, bool NT, bool CENTER>
__device__ __forceinline__ void qk_tile(const StatsPackParams& p, const Tile& T, int64_t rz,
                                        int64_t rank, uint8_t* send, const uint4* x,
                                        const uint4& m, int cb, Phase0Lds& lds) {
    constexpr int CPB = 256, HPB = CPB / D, PPH = D / 8;
    constexpr int HEAD_MASK = (PPH - 1) | 32;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t H = p.H, h = p.h, L = p.L;

    // Amax of this thread's rows, |fp32(q)| or |RN(fp32(k) - fp32(mean))| (>= 0, so an
    // empty range leaves 0 and the floor decides), then over the head's lanes and waves.
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (T.rq + 8 * i < T.namax) {
            float f[8];
            decode8<DT>(x[i], f);
            if constexpr (CENTER) {
                float mf[8];
                decode8<DT>(m, mf);
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaxf(a, __builtin_fabsf(f[e] - mf[e]));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaxf(a, __builtin_fabsf(f[e]));
            }
        }
    }
    a = wave_max_xor<HEAD_MASK>(a);
    auto& red = lds.red;
    if ((lane & HEAD_MASK) == 0) red[wave][T.hib] = a;
    __syncthreads();
    const float amax = fmaxf(kFloor, fmaxf(fmaxf(red[0][T.hib], red[1][T.hib]),
                                           fmaxf(red[2][T.hib], red[3][T.hib])));
    const bool scale_writer = wave == 0 && (lane & HEAD_MASK) == 0 && T.valid;
    const int64_t arank = rz * p.amax_rank_stride;
    if (scale_writer) (CENTER ? p.k_amax : p.q_amax)[arank + (T.b * H + T.head) * p.slots + T.j] = amax;

    // First and last slot: per-channel raw min/max over the live rows (zeros as +0;
    // (+inf, -inf) when the rank has no live row in the group): each thread reduces its
    // rows (both extremes in one pass over them), a [row lane][channel] LDS table the row
    // lanes, min then max.
    if (T.j == 0 || T.j == T.n - 1) {
        const bool mm_live = min(T.hi, p.used) > T.lo;
        float rmin[8], rmax[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            rmin[e] = __builtin_inff();
            rmax[e] = -__builtin_inff();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (T.rq + 8 * i < T.namax) {
                float f[8];
                decode8<DT>(x[i], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rmin[e] = fminf(rmin[e], f[e] + 0.0f);
                    rmax[e] = fmaxf(rmax[e], f[e] + 0.0f);
                }
            }
        }
        auto& col = lds.col;
        const int64_t ch0 = (int64_t)cb * CPB;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            if (mm_live) {
#pragma unroll
                for (int e = 0; e < 8; ++e) col[T.rq][T.cq * 8 + e] = w ? rmax[e] : rmin[e];
            }
            __syncthreads();
            if (ch0 + tid < H * D) {
                // thread tid reduces channel tid of the workgroup's 256
                float v = w ? -__builtin_inff() : __builtin_inff();
                if (mm_live) {
#pragma unroll
                    for (int rr = 0; rr < 8; ++rr)
                        v = w ? fmaxf(v, col[rr][tid]) : fminf(v, col[rr][tid]);
                }
                const int64_t hd = (int64_t)cb * HPB + tid / D;
                float* mm = (CENTER ? p.k_minmax : p.q_minmax) + rz * p.minmax_rank_stride;
                for (int e2 = 0; e2 < 2; ++e2) {
                    if ((e2 == 0 && T.j != 0) || (e2 == 1 && T.j != T.n - 1)) continue;
                    mm[((T.b * H + hd) * 2 + e2) * 2 * D + w * D + tid % D] = v;
                }
            }
            __syncthreads();
        }
    }
    if (waits_for_derive(rank, L, p.S, p.used, T.j, T.n)) return;

    // Quantize every row of the rank in the group (rows in the zero tail included), two
    // rows of 8 channels per call.
    const QuantScale sc = make_scale(amax);
    const int64_t dst = T.head / h, jl = T.head % h;
    uint8_t* chunk = send + dst * p.dest_stride;
    const int64_t os = h * D;                                       // row stride of a section
    uint8_t* out0 = chunk + (CENTER ? p.sec : 0) + ((T.b * L + T.l0) * h + jl) * D + T.pc * 8;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint4 c = quantize16<DT, CENTER, CENTER || DT == kBF16>(x[i], x[i + 1], m, m, sc);
        uint8_t* o = out0 + (T.rq + 8 * i) * os;
        if (T.valid && T.rq + 8 * i < T.nrow) store8<NT>(o, c.x, c.y);
        if (T.valid && T.rq + 8 * i + 8 < T.nrow) store8<NT>(o + 8 * os, c.z, c.w);
    }
    if (scale_writer) {
        float* s = reinterpret_cast<float*>(chunk + 3 * p.sec + (CENTER ? p.ssec : 0)) +
                   (T.b * h + jl) * p.slots;
        s[T.j] = sc.s;
    }
}

template <int DT, int D, bool NT, bool VS>
__global__ __launch_bounds__(kThreads) void stats_pack0_kernel(StatsPackParams p) {
    constexpr int CPB = 256, HPB = CPB / D, PPH = D / 8;
    const int64_t L = p.L, H = p.H, h = p.h;
    const int64_t rz = blockIdx.z, rank = p.rank0 + rz;
    uint8_t* send = p.send + rz * p.send_rank_stride;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    if (blockIdx.x == 0) {
        // Zero the padding bytes after each section of every destination chunk.
        const int64_t data = p.B * L * h * D;          // bytes of each code section
        const int64_t sdata = 4 * p.B * h * p.slots;   // bytes of each scale section
        for (int64_t i = tid; i < p.P * 5 * 256; i += kThreads) {
            const int64_t dst = i / (5 * 256), sect = (i / 256) % 5, off = i % 256;
            const int64_t start = sect < 3 ? sect * p.sec + data
                                           : 3 * p.sec + (sect - 3) * p.ssec + sdata;
            const int64_t end = sect < 3 ? (sect + 1) * p.sec : 3 * p.sec + (sect - 2) * p.ssec;
            if (start + off < end) send[dst * p.dest_stride + start + off] = 0;
        }
    }

    // Workgroup (b, slot, channel block, tensor), tensors fastest: the workgroups in
    // flight read the same rows and channels of Q, K and V, and together whole rows
    // (measured 3 % faster than channel blocks fastest on the long workload).
    int bid = blockIdx.x;
    const int t = bid % 3;
    bid /= 3;
    const int cb = bid % p.nhb;
    bid /= p.nhb;
    Tile T;
    T.j = bid % p.grid_slots;
    T.b = bid / p.grid_slots;
    const int64_t g0 = first_group(rank, L);
    T.n = last_group(rank, L) - g0 + 1;
    const int64_t HD = H * D;

    if (T.j >= T.n) {
        // A slot this rank never touches: the floor, and its scale passed through as the
        // pack passes every slot's amax.
        const int64_t head = (int64_t)cb * HPB + tid;
        if (t < 2 && tid < HPB && head < H) {
            const int64_t dst = head / h, jl = head % h;
            (t ? p.k_amax : p.q_amax)[rz * p.amax_rank_stride + (T.b * H + head) * p.slots + T.j] =
                kFloor;
            float* s = reinterpret_cast<float*>(send + dst * p.dest_stride + 3 * p.sec +
                                                (t ? p.ssec : 0)) + (T.b * h + jl) * p.slots;
            s[T.j] = kFloor / 127.0f;
        }
        return;
    }

    T.cq = lane & 31;
    T.rq = wave * 2 + (lane >> 5);
    T.valid = (int64_t)cb * CPB + T.cq * 8 < HD;
    // A ragged block's lanes past the row read (and never store) the piece 16 lanes down.
    const int cqa = T.valid ? T.cq : T.cq - 16;
    T.hib = T.cq / PPH;
    T.pc = cqa % PPH;
    T.head = (int64_t)cb * HPB + cqa / PPH;
    T.g = g0 + T.j;
    T.lo = max(kGroup * T.g, rank * L);
    T.hi = min(kGroup * T.g + kGroup, rank * L + L);
    T.nrow = (int)(T.hi - T.lo);                               // 1..64 rows of this rank
    // The grouped amax of the one group that mixes live rows and the zero tail runs over
    // its live rows only; the min/max runs over the live rows (the same rows, or none).
    const int64_t amax_hi =
        (p.used < p.S && T.g == (p.used - 1) / kGroup) ? min(T.hi, p.used) : T.hi;
    T.namax = (int)(amax_hi - T.lo);                           // may be <= 0
    T.l0 = T.lo - rank * L;                                    // local row of the first row

    // Issue every load first: eight rows of the tensor, 16 bytes each (and the K mean, or
    // the V scale).  V is always streamed (read once, never again in the step), Q and K
    // where the launch streams.  Rows past the range re-read the last row (no load sits
    // in a branch, so all are in flight together).
    const uint64_t x0 = (uint64_t)rz * p.x_rank_stride +
                        (uint64_t)(((T.b * L + T.l0) * H + T.head) * D + T.pc * 8);
    uint4 x[8], m = make_uint4(0u, 0u, 0u, 0u);
    if (t == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            x[i] = load16<true>(p.v + x0 + (uint64_t)(min(T.rq + 8 * i, T.nrow - 1) * HD));
    } else {
        // (streamed Q/K loads: 1 % faster on the long workload and 8 % on
        // video_dit_aligned than cached ones)
        const uint16_t* src = t ? p.k : p.q;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            x[i] = load16<NT>(src + x0 + (uint64_t)(min(T.rq + 8 * i, T.nrow - 1) * HD));
        if (t == 1) m = load16(p.mean + (T.b * H + T.head) * D + T.pc * 8);
    }
    float4 sv[4];
    if constexpr (VS) {
        if (t == 2) {
            // the 8 channels' V divisors, twice (the conversion takes two rows of 8 channels)
            const float4* vp =
                reinterpret_cast<const float4*>(p.v_scale + (T.b * H + T.head) * D + T.pc * 8);
            sv[0] = vp[0];
            sv[1] = vp[1];
            sv[2] = sv[0];
            sv[3] = sv[1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    __shared__ Phase0Lds lds;
    if (t == 0) {
        qk_tile<DT, D, NT, false>(p, T, rz, rank, send, x, m, cb, lds);
    } else if (t == 1) {
        qk_tile<DT, D, NT, true>(p, T, rz, rank, send, x, m, cb, lds);
    } else {
        // V needs no statistic: E4M3 of every row of the rank in the group, two rows of 8
        // channels per conversion.
        const int64_t dst = T.head / h, jl = T.head % h;
        const int64_t os = h * D;
        uint8_t* out0 = send + dst * p.dest_stride + 2 * p.sec +
                        ((T.b * L + T.l0) * h + jl) * D + T.pc * 8;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            uint4 e;
            if constexpr (VS)
                e = e4m3x16_scaled<DT>(x[i], x[i + 1], sv);
            else
                e = e4m3x16<DT>(x[i], x[i + 1]);
            uint8_t* o = out0 + (T.rq + 8 * i) * os;
            if (T.valid && T.rq + 8 * i < T.nrow) store8<NT>(o, e.x, e.y);
            if (T.valid && T.rq + 8 * i + 8 < T.nrow) store8<NT>(o + 8 * os, e.z, e.w);
        }
    }
}

// Phase 1: derive of the rank's first and last slot for Q and K, and the pack of the slots
// that waited for it.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void derive_pack_kernel(StatsPackParams p) {
    constexpr int HPB = 128 / D;             // heads per workgroup (128 channels)
    constexpr int PPH = D / 8;               // 16-byte pieces (8 channels) per head row
    // Lane layout: 16 consecutive 16-byte pieces (the workgroup's 256 bytes of a row) x 4
    // rows per wave.
    constexpr int HEAD_MASK = D == 128 ? 63 : 55;
    const int64_t L = p.L, H = p.H, h = p.h;
    const int64_t rz = blockIdx.z, rank = p.rank0 + rz;
    uint8_t* send = p.send + rz * p.send_rank_stride;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    int bid = blockIdx.x;
    const int hb = bid % p.nhb;
    bid /= p.nhb;
    const int jg = bid % p.grid_slots;
    const int64_t b = bid / p.grid_slots;
    const int64_t g0 = first_group(rank, L);
    const int64_t n = last_group(rank, L) - g0 + 1;
    if (jg == 1 && n == 1) return;   // one touched slot: the jg = 0 workgroup has it
    const int64_t j = jg == 0 ? 0 : n - 1;
    const bool wait = waits_for_derive(rank, L, p.S, p.used, j, n);
    const int64_t arank = rz * p.amax_rank_stride;

    const int cq = lane & 15;                  // 16-byte piece of the workgroup's row
    const int rq = wave * 4 + (lane >> 4);     // row lane 0..15: rows rq + 16 i, i < 4
    const int hib = cq / PPH, pc = cq % PPH;
    const int64_t head = (int64_t)hb * HPB + hib;
    const int64_t dst = head / h, jl = head % h;
    const int64_t g = g0 + j;
    const int64_t lo = max(kGroup * g, rank * L), hi = min(kGroup * g + kGroup, rank * L + L);
    const int nrow = (int)(hi - lo);                       // 1..64 rows of this rank
    const int64_t l0 = lo - rank * L;                      // local row of the first row

    // The waiting slot's rows of Q and K and the K mean, loaded before the derive.
    const int64_t xs = H * D;                              // row stride of the shards
    const uint64_t x0 = (uint64_t)rz * p.x_rank_stride +
                        (uint64_t)(((b * L + l0) * H + head) * D + pc * 8);
    uint4 qv[4], kv[4], m;
    if (wait) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t o = x0 + (uint64_t)(min(rq + 16 * i, nrow - 1) * xs);
            qv[i] = load16(p.q + o);
            kv[i] = load16(p.k + o);
        }
        m = load16(p.mean + (b * H + head) * D + pc * 8);
    }
    __builtin_amdgcn_sched_barrier(0);

    // derive_k_boundary_amax (description) for this slot, both tensors, every head of the
    // block: the max over the ranks touching the group of max(1e-7, max_d max(RN(max - m),
    // RN(m - min))) of their gathered min/max (m = +0 for Q).  Thread (tensor t, channel c)
    // first takes its channel's max over the touching ranks; the max over channels and the
    // floor follow (max is exact and order-free, so this is the same value).
    const int t = tid >> 7, cc = tid & 127, hd = cc / D, d = cc % D;
    const int64_t dhead = (int64_t)hb * HPB + hd;
    const float mref = t ? decode1<DT>(p.mean[(b * H + dhead) * D + d]) : 0.0f;
    const float* mm = t ? p.k_minmax : p.q_minmax;
    float v = -__builtin_inff();
    for (int64_t r = 0; r < p.P; ++r) {
        if (!(r * L < kGroup * g + kGroup && kGroup * g < r * L + L)) continue;
        const int er = g == first_group(r, L) ? 0 : 1;
        const float* base = mm + r * p.gathered_stride + (((b * H + dhead) * 2 + er) * 2) * D;
        v = fmaxf(v, fmaxf(base[D + d] - mref, mref - base[d]));
    }
    v = wave_max_xor<63>(v);
    __shared__ float dred[4];
    if (lane == 0) dred[wave] = v;
    __syncthreads();
    // wave w holds channels [64 (w & 1), 64 (w & 1) + 64) of tensor w >> 1
    const float qd = D == 128 ? fmaxf(dred[0], dred[1]) : dred[hib];
    const float kd = D == 128 ? fmaxf(dred[2], dred[3]) : dred[2 + hib];
    const float qamax = fmaxf(kFloor, qd);
    const float kamax = fmaxf(kFloor, kd);
    if (tid < 2 * HPB) {
        const int tt = tid / HPB, hh = tid % HPB;
        const float a = fmaxf(kFloor, D == 128 ? fmaxf(dred[2 * tt], dred[2 * tt + 1])
                                               : dred[2 * tt + hh]);
        (tt ? p.k_amax : p.q_amax)[arank + (b * H + (int64_t)hb * HPB + hh) * p.slots + j] = a;
    }
    if (!wait) return;

    // Quantize every row of the rank in the group (rows in the zero tail included), two
    // rows of 8 channels per call.
    uint8_t* chunk = send + dst * p.dest_stride;
    uint8_t* out0 = chunk + ((b * L + l0) * h + jl) * D + pc * 8;    // the group's first row
    const int64_t os = h * D;                                       // row stride of a section
    const QuantScale sq = make_scale(qamax);
    const QuantScale sk = make_scale(kamax);
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        const uint4 cqv = quantize16<DT, false, DT == kBF16>(qv[i], qv[i + 1], m, m, sq);
        const uint4 ckv = quantize16<DT, true, true>(kv[i], kv[i + 1], m, m, sk);
        uint8_t* o = out0 + (rq + 16 * i) * os;
        if (rq + 16 * i < nrow) {
            store8<false>(o, cqv.x, cqv.y);
            store8<false>(o + p.sec, ckv.x, ckv.y);
        }
        if (rq + 16 * i + 16 < nrow) {
            store8<false>(o + 16 * os, cqv.z, cqv.w);
            store8<false>(o + 16 * os + p.sec, ckv.z, ckv.w);
        }
    }
    if (wave == 0 && (lane & HEAD_MASK) == 0) {               // one thread per head
        float* qs = reinterpret_cast<float*>(chunk + 3 * p.sec) + (b * h + jl) * p.slots;
        float* ks = reinterpret_cast<float*>(chunk + 3 * p.sec + p.ssec) + (b * h + jl) * p.slots;
        qs[j] = sq.s;
        ks[j] = sk.s;
    }
}

template <int DT, int D, int PHASE>
hipError_t launch_t(const StatsPackLaunch& a, hipStream_t stream) {
    StatsPackParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.mean = a.mean;
    p.v_scale = a.v_scale;
    p.q_amax = a.q_amax;
    p.k_amax = a.k_amax;
    p.q_minmax = a.q_minmax;
    p.k_minmax = a.k_minmax;
    p.send = a.send;
    p.dest_stride = a.dest_stride;
    p.x_rank_stride = a.x_rank_stride;
    p.amax_rank_stride = a.amax_rank_stride;
    p.minmax_rank_stride = a.minmax_rank_stride;
    p.send_rank_stride = a.send_rank_stride;
    p.gathered_stride = a.B * a.H * 4 * D;
    p.B = a.B;
    p.L = a.L;
    p.H = a.H;
    p.h = a.H / a.P;
    p.P = a.P;
    p.S = a.P * a.L;
    p.used = a.used;
    p.slots = slots_of(a.L);
    p.sec = chunk_section(a.B, a.L, p.h, D);
    p.ssec = chunk_scale_section(a.B, a.L, p.h);
    p.rank0 = a.rank0;
    const dim3 block(kThreads);
    if constexpr (PHASE == 0) {
        p.nhb = (int)((a.H * D + 255) / 256);
        p.grid_slots = (int)p.slots;
        const int64_t written = a.nranks * 3 * a.B * a.L * a.H * D;   // code bytes
        const bool nt = written > kResidentBytes;
        const dim3 grid((unsigned)(a.B * p.slots * p.nhb * 3), 1, (unsigned)a.nranks);
        if (a.v_scale) {
            if (nt) hipLaunchKernelGGL((stats_pack0_kernel<DT, D, true, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((stats_pack0_kernel<DT, D, false, true>), grid, block, 0, stream, p);
        } else {
            if (nt) hipLaunchKernelGGL((stats_pack0_kernel<DT, D, true, false>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((stats_pack0_kernel<DT, D, false, false>), grid, block, 0, stream, p);
        }
    } else {
        p.nhb = (int)(a.H * D / 128);
        p.grid_slots = 2;
        const dim3 grid((unsigned)(a.B * 2 * p.nhb), 1, (unsigned)a.nranks);
        hipLaunchKernelGGL((derive_pack_kernel<DT, D>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <int PHASE>
hipError_t launch_phase(const StatsPackLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64, PHASE>(a, stream)
                                           : launch_t<kBF16, 128, PHASE>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64, PHASE>(a, stream)
                     : launch_t<kFP16, 128, PHASE>(a, stream);
}

}  // namespace

hipError_t launch_stats_pack(const StatsPackLaunch& a, hipStream_t stream) {
    return a.phase == 0 ? launch_phase<0>(a, stream) : launch_phase<1>(a, stream);
}

}  // namespace ulp
