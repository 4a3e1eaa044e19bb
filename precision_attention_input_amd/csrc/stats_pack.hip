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
// Phase 0: one 256-thread workgroup per (rank, b, slot, 128 channels: one head at D = 128,
// two at D = 64) loads the rank's rows of the group (at most 64, four per thread) of Q and
// K once, reduces the raw |Q| and centered |K - mean| amax of each head (and, for the first
// and last slot, the per-channel raw min/max) in the same registers, writes them, and
// quantizes Q and K with the new scales, unless the slot must wait for derive.  V, which
// needs no statistic, is converted in the same launch: by the same workgroups from their
// own rows when the launch's data fits the cache, by workgroups of its own in the pack
// kernel's layout when it streams from HBM.  Phase 1, after the min/max are gathered: one
// workgroup per (rank, b, first or last slot, 128 channels) derives the slot's amax for Q
// and K as derive_k_boundary_amax (description) does, writes it, and, if the slot waited,
// re-reads its rows and quantizes them with it.  The outputs are bit-identical to the
// separate statistics, derive and pack launches: the same amax (a direct max of the same
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
    int rank0, nhb, grid_slots;
    int n_qk, v_row_blocks, v_col_blocks;   // phase 0: V workgroups follow the n_qk others
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

template <int DT, int D, int PHASE, bool NT, bool VS>
__global__ __launch_bounds__(kThreads) void stats_pack_kernel(StatsPackParams p) {
    constexpr int HPB = 128 / D;             // heads per workgroup (128 channels)
    constexpr int PPH = D / 8;               // 16-byte pieces (8 channels) per head row
    // Lane layout: 16 consecutive 16-byte pieces (the workgroup's 256 bytes of a row) x 4
    // rows per wave, so every load instruction reads whole cache lines of 4 rows.  Lanes of
    // one head differ in the piece bits (0-3 at D = 128, 0-2 at D = 64) and the row bits 4-5.
    constexpr int HEAD_MASK = D == 128 ? 63 : 55;
    const int64_t L = p.L, H = p.H, h = p.h;
    const int64_t rz = blockIdx.z, rank = p.rank0 + rz;
    uint8_t* send = p.send + rz * p.send_rank_stride;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    if (PHASE == 0 && blockIdx.x == 0) {
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

    // Where the launch streams from HBM, V goes through workgroups of its own (after the
    // statistics workgroups) in the pack kernel's layout; in smaller launches, whose data
    // the cache holds, the statistics workgroups convert it with their own rows.  Each
    // choice measured 2-8 % faster than the other at its sizes.
    constexpr bool V_SPLIT = NT;
    constexpr bool V_HERE = PHASE == 0 && !V_SPLIT;
    if (PHASE == 0 && V_SPLIT && (int)blockIdx.x >= p.n_qk) {
        // V needs no statistic: the pack kernel's layout, 8 rows x 32 sixteen-element
        // vectors per workgroup, column blocks fastest (whole rows in flight).
        constexpr int VPH = D / 16;
        const uint32_t vbid = blockIdx.x - (uint32_t)p.n_qk;
        const uint32_t cblk = vbid % (uint32_t)p.v_col_blocks;
        const uint32_t rblk = vbid / (uint32_t)p.v_col_blocks;
        const uint32_t bb = rblk / (uint32_t)p.v_row_blocks;
        const uint32_t l = (rblk % (uint32_t)p.v_row_blocks) * 8 + tid / 32;
        const uint32_t col = cblk * 32 + tid % 32;
        if (l >= (uint32_t)L || col >= (uint32_t)(H * VPH)) return;
        const uint32_t vhead = col / VPH, vdv = col % VPH;
        const uint64_t xo = (uint64_t)rz * p.x_rank_stride +
                            ((uint64_t)bb * L + l) * (uint64_t)(H * D) + col * 16;
        const uint4 v0 = load16<true>(p.v + xo);
        const uint4 v1 = load16<true>(p.v + xo + 8);
        uint8_t* o = send + (int64_t)(vhead / h) * p.dest_stride + 2 * p.sec +
                     (((int64_t)bb * L + l) * h + vhead % h) * D + vdv * 16;
        if constexpr (VS) {
            const float4* vp = reinterpret_cast<const float4*>(
                p.v_scale + ((int64_t)bb * H + vhead) * D + vdv * 16);
            float4 sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = vp[i];
            store16<NT>(o, e4m3x16_scaled<DT>(v0, v1, sv));
        } else {
            store16<NT>(o, e4m3x16<DT>(v0, v1));
        }
        return;
    }

    // Workgroup: head block fastest, so the workgroups in flight cover whole rows.
    int bid = blockIdx.x;
    const int hb = bid % p.nhb;
    bid /= p.nhb;
    const int jg = bid % p.grid_slots;
    const int64_t b = bid / p.grid_slots;
    const int64_t g0 = first_group(rank, L);
    const int64_t n = last_group(rank, L) - g0 + 1;
    int64_t j = jg;
    if (PHASE == 1) {
        if (jg == 1 && n == 1) return;   // one touched slot: the jg = 0 workgroup has it
        j = jg == 0 ? 0 : n - 1;
    }
    const bool wait = waits_for_derive(rank, L, p.S, p.used, j, n);
    const int64_t arank = rz * p.amax_rank_stride;

    if (PHASE == 0 && j >= n) {
        // A slot this rank never touches: the floor, and its scale passed through as the
        // pack passes every slot's amax.
        if (tid < HPB) {
            const int64_t head = (int64_t)hb * HPB + tid;
            const int64_t dst = head / h, jl = head % h;
            p.q_amax[arank + (b * H + head) * p.slots + j] = kFloor;
            p.k_amax[arank + (b * H + head) * p.slots + j] = kFloor;
            uint8_t* chunk = send + dst * p.dest_stride;
            float* qs = reinterpret_cast<float*>(chunk + 3 * p.sec) + (b * h + jl) * p.slots;
            float* ks = reinterpret_cast<float*>(chunk + 3 * p.sec + p.ssec) +
                        (b * h + jl) * p.slots;
            qs[j] = kFloor / 127.0f;
            ks[j] = kFloor / 127.0f;
        }
        return;
    }

    const int cq = lane & 15;                  // 16-byte piece of the workgroup's row
    const int rq = wave * 4 + (lane >> 4);     // row lane 0..15: rows rq + 16 i, i < 4
    const int hib = cq / PPH, pc = cq % PPH;
    const int64_t head = (int64_t)hb * HPB + hib;
    const int64_t dst = head / h, jl = head % h;
    const int64_t g = g0 + j;
    const int64_t lo = max(kGroup * g, rank * L), hi = min(kGroup * g + kGroup, rank * L + L);
    const int nrow = (int)(hi - lo);                       // 1..64 rows of this rank
    // The grouped amax of the one group that mixes live rows and the zero tail runs over
    // its live rows only; the min/max runs over the live rows (the same rows, or none).
    const int64_t amax_hi =
        (p.used < p.S && g == (p.used - 1) / kGroup) ? min(hi, p.used) : hi;
    const int namax = (int)(amax_hi - lo);                 // may be <= 0
    const int64_t l0 = lo - rank * L;                      // local row of the first row

    // Issue every load first: four rows of Q and K (and of V where these workgroups convert
    // it), 16 bytes each, and the K mean.  Rows past the range re-read the last row (no load
    // sits in a branch, so all are in flight together).
    const int64_t xs = H * D;                              // row stride of the shards
    const uint64_t x0 = (uint64_t)rz * p.x_rank_stride +
                        (uint64_t)(((b * L + l0) * H + head) * D + pc * 8);
    uint4 qv[4], kv[4], vv[4], m;
    if (PHASE == 0 || wait) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t o = x0 + (uint64_t)(min(rq + 16 * i, nrow - 1) * xs);
            qv[i] = load16(p.q + o);
            kv[i] = load16(p.k + o);
            if constexpr (V_HERE) vv[i] = load16<true>(p.v + o);
        }
        m = load16(p.mean + (b * H + head) * D + pc * 8);
    }
    float4 sv[4];
    if constexpr (V_HERE && VS) {
        // the 8 channels' V divisors, twice (the conversion takes two rows of 8 channels)
        const float4* vp =
            reinterpret_cast<const float4*>(p.v_scale + (b * H + head) * D + pc * 8);
        sv[0] = vp[0];
        sv[1] = vp[1];
        sv[2] = sv[0];
        sv[3] = sv[1];
    }
    __builtin_amdgcn_sched_barrier(0);

    uint8_t* chunk = send + dst * p.dest_stride;
    uint8_t* out0 = chunk + ((b * L + l0) * h + jl) * D + pc * 8;    // the group's first row
    const int64_t os = h * D;                                       // row stride of a section
    const bool scale_writer = wave == 0 && (lane & HEAD_MASK) == 0;  // one thread per head

    float qamax, kamax;
    if constexpr (PHASE == 0) {
        if constexpr (V_HERE) {
            // V needs no statistic: convert and store it first, which frees its registers.
            // Each conversion takes two rows of this thread's 8 channels.
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                uint4 e;
                if constexpr (VS)
                    e = e4m3x16_scaled<DT>(vv[i], vv[i + 1], sv);
                else
                    e = e4m3x16<DT>(vv[i], vv[i + 1]);
                uint8_t* o = out0 + 2 * p.sec + (rq + 16 * i) * os;
                if (rq + 16 * i < nrow) store8<NT>(o, e.x, e.y);
                if (rq + 16 * i + 16 < nrow) store8<NT>(o + 16 * os, e.z, e.w);
            }
        }

        // Amax of this thread's rows, |fp32(q)| and |RN(fp32(k) - fp32(mean))| (>= 0, so an
        // empty range leaves 0 and the floor decides), then over the head's lanes and waves.
        float qa = 0.0f, ka = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (rq + 16 * i < namax) {
                float f[8], mf[8];
                decode8<DT>(qv[i], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) qa = fmaxf(qa, __builtin_fabsf(f[e]));
                decode8<DT>(kv[i], f);
                decode8<DT>(m, mf);
#pragma unroll
                for (int e = 0; e < 8; ++e) ka = fmaxf(ka, __builtin_fabsf(f[e] - mf[e]));
            }
        }
        qa = wave_max_xor<HEAD_MASK>(qa);
        ka = wave_max_xor<HEAD_MASK>(ka);
        __shared__ float red[4][2][HPB];                    // [wave][tensor][head]
        if ((lane & HEAD_MASK) == 0) {
            red[wave][0][hib] = qa;
            red[wave][1][hib] = ka;
        }
        __syncthreads();
        qamax = fmaxf(kFloor, fmaxf(fmaxf(red[0][0][hib], red[1][0][hib]),
                                    fmaxf(red[2][0][hib], red[3][0][hib])));
        kamax = fmaxf(kFloor, fmaxf(fmaxf(red[0][1][hib], red[1][1][hib]),
                                    fmaxf(red[2][1][hib], red[3][1][hib])));
        if (scale_writer) {
            p.q_amax[arank + (b * H + head) * p.slots + j] = qamax;
            p.k_amax[arank + (b * H + head) * p.slots + j] = kamax;
        }

        // First and last slot: per-channel raw min/max over the live rows (zeros as +0;
        // (+inf, -inf) when the rank has no live row in the group): each thread reduces its
        // rows, a [row lane][channel] LDS table the row lanes, one (tensor, min or max) at
        // a time.
        if (j == 0 || j == n - 1) {
            const bool mm_live = min(hi, p.used) > lo;
            __shared__ float col[16][129];
#pragma unroll 1
            for (int pass = 0; pass < 4; ++pass) {
                const int t = pass >> 1, w = pass & 1;
                if (mm_live) {
                    float r[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = w ? -__builtin_inff() : __builtin_inff();
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (rq + 16 * i < namax) {
                            float f[8];
                            decode8<DT>(t ? kv[i] : qv[i], f);
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                r[e] = w ? fmaxf(r[e], f[e] + 0.0f) : fminf(r[e], f[e] + 0.0f);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) col[rq][cq * 8 + e] = r[e];
                }
                __syncthreads();
                if (tid < 128) {
                    // thread tid reduces channel tid of the workgroup's 128
                    float a = w ? -__builtin_inff() : __builtin_inff();
                    if (mm_live) {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr)
                            a = w ? fmaxf(a, col[rr][tid]) : fminf(a, col[rr][tid]);
                    }
                    const int64_t hd = (int64_t)hb * HPB + tid / D;
                    float* mm = (t ? p.k_minmax : p.q_minmax) + rz * p.minmax_rank_stride;
                    for (int e2 = 0; e2 < 2; ++e2) {
                        if ((e2 == 0 && j != 0) || (e2 == 1 && j != n - 1)) continue;
                        mm[((b * H + hd) * 2 + e2) * 2 * D + w * D + tid % D] = a;
                    }
                }
                __syncthreads();
            }
        }
        if (wait) return;
    } else {
        // derive_k_boundary_amax (description) for this slot, both tensors, every head of
        // the block: the max over the ranks touching the group of max(1e-7, max_d
        // max(RN(max - m), RN(m - min))) of their gathered min/max (m = +0 for Q).  Thread
        // (tensor t, channel c) first takes its channel's max over the touching ranks; the
        // max over channels and the floor follow (max is exact and order-free, so this is
        // the same value).
        const int t = tid >> 7, cc = tid & 127, hd = cc / D, d = cc % D;
        const int64_t dhead = (int64_t)hb * HPB + hd;
        const float mref =
            t ? decode1<DT>(p.mean[(b * H + dhead) * D + d]) : 0.0f;
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
        qamax = fmaxf(kFloor, qd);
        kamax = fmaxf(kFloor, kd);
        if (tid < 2 * HPB) {
            const int tt = tid / HPB, hh = tid % HPB;
            const float a = fmaxf(kFloor, D == 128 ? fmaxf(dred[2 * tt], dred[2 * tt + 1])
                                                   : dred[2 * tt + hh]);
            (tt ? p.k_amax : p.q_amax)[arank + (b * H + (int64_t)hb * HPB + hh) * p.slots + j] = a;
        }
        if (!wait) return;
    }

    // Quantize every row of the rank in the group (rows in the zero tail included), two
    // rows of 8 channels per call.
    const QuantScale sq = make_scale(qamax);
    const QuantScale sk = make_scale(kamax);
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        const uint4 cqv = quantize16<DT, false, DT == kBF16>(qv[i], qv[i + 1], m, m, sq);
        const uint4 ckv = quantize16<DT, true, true>(kv[i], kv[i + 1], m, m, sk);
        uint8_t* o = out0 + (rq + 16 * i) * os;
        if (rq + 16 * i < nrow) {
            store8<NT>(o, cqv.x, cqv.y);
            store8<NT>(o + p.sec, ckv.x, ckv.y);
        }
        if (rq + 16 * i + 16 < nrow) {
            store8<NT>(o + 16 * os, cqv.z, cqv.w);
            store8<NT>(o + 16 * os + p.sec, ckv.z, ckv.w);
        }
    }
    if (scale_writer) {
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
    p.nhb = (int)(a.H * D / 128);
    p.grid_slots = PHASE == 0 ? (int)p.slots : 2;
    p.n_qk = (int)(a.B * p.grid_slots * p.nhb);
    p.v_row_blocks = (int)((a.L + 7) / 8);
    p.v_col_blocks = (int)((a.H * D / 16 + 31) / 32);
    const dim3 block(kThreads);
    if constexpr (PHASE == 0) {
        const int64_t written = a.nranks * 3 * a.B * a.L * a.H * D;   // code bytes
        const bool nt = written > kResidentBytes;
        // V workgroups of their own in the streaming instantiation (see the kernel)
        const int64_t n_v = nt ? a.B * p.v_row_blocks * p.v_col_blocks : 0;
        const dim3 grid((unsigned)(p.n_qk + n_v), 1, (unsigned)a.nranks);
        if (a.v_scale) {
            if (nt) hipLaunchKernelGGL((stats_pack_kernel<DT, D, 0, true, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((stats_pack_kernel<DT, D, 0, false, true>), grid, block, 0, stream, p);
        } else {
            if (nt) hipLaunchKernelGGL((stats_pack_kernel<DT, D, 0, true, false>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((stats_pack_kernel<DT, D, 0, false, false>), grid, block, 0, stream, p);
        }
    } else {
        const dim3 grid((unsigned)p.n_qk, 1, (unsigned)a.nranks);
        hipLaunchKernelGGL((stats_pack_kernel<DT, D, 1, false, false>), grid, block, 0, stream, p);
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
