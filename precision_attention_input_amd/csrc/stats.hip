// stats.hip -- per-rank statistics over 64-row global groups (gfx950).
//
//  * grouped amax: flashinfer.comm._ulysses_lowp.k_grouped_amax (description, Returns):
//    for every global group a rank touches, max over the rank's rows of the group and all
//    channels of |RN(fp32(x) - fp32(mean))|, floored at 1e-7; the one group mixing live
//    rows and zero padding is taken over its live rows only.
//  * boundary min/max: the per-channel raw min/max over the live rows of the rank's first
//    and last touched group, which derive_k_boundary_amax (description) consumes.
//
// One 256-thread workgroup handles one (rank, tensor, b, slot, head block): at most 64 rows
// x (256 / D) heads, i.e. 32 sixteen-byte vectors per row and 8 rows in flight, each thread
// issuing its (up to) 8 loads before reducing.  Per channel a thread keeps only the raw
// extremes of its rows (three packed 16-bit integer operations per two values, Order16);
// the amax then follows from them by the identity that derive_k_boundary_amax
// (description) rests on, max |RN(x - m)| = max(RN(max x - m), RN(m - min x)), so the
// per-element work is the same for the amax and the min/max, and both come out of the
// same pass: the fused group entry point reads Q and K exactly once.
#include "order16.h"
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

struct StatsParams {
    const uint16_t* x[2];
    const uint16_t* mean[2];
    float* amax[2];
    float* minmax[2];
    int64_t x_rank_stride, amax_rank_stride, minmax_rank_stride;
    int64_t L, H, S, used, slots;
    int rank0, nhb, grid_slots;
    int boundary_only;            // grid covers slot 0 and slot n-1 only (min/max alone)
};

template <int DT, int D, bool NT>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsParams p) {
    constexpr int VPH = D / 8;       // 16-byte vectors per head row
    constexpr int HB = 256 / D;      // heads per workgroup: 32 vectors per row
    const int tensor = blockIdx.y;
    const uint16_t* x = p.x[tensor];
    if (x == nullptr) return;
    const int64_t L = p.L, H = p.H;
    const int64_t rank = p.rank0 + blockIdx.z;
    int bid = blockIdx.x;
    const int hb = bid % p.nhb;
    bid /= p.nhb;
    const int jg = bid % p.grid_slots;
    const int64_t b = bid / p.grid_slots;

    const int64_t g0 = first_group(rank, L);
    const int64_t n = last_group(rank, L) - g0 + 1;
    int64_t j = jg;
    if (p.boundary_only) {              // slot 0 and slot n-1 of every rank
        if (jg == 1 && n == 1) return;
        j = jg == 0 ? 0 : n - 1;
    }
    float* amax_out = p.amax[tensor] ? p.amax[tensor] + blockIdx.z * p.amax_rank_stride : nullptr;
    float* mm_out =
        p.minmax[tensor] ? p.minmax[tensor] + blockIdx.z * p.minmax_rank_stride : nullptr;

    const int tid = threadIdx.x;
    if (j >= n) {                       // a slot this rank never touches: the floor
        if (amax_out && tid < HB && (int64_t)hb * HB + tid < H)
            amax_out[(b * H + hb * HB + tid) * p.slots + j] = kFloor;
        return;
    }

    const int c = tid & 31, rl = tid >> 5;
    const int hib = c / VPH, dv = c % VPH;
    const int64_t head = (int64_t)hb * HB + hib;
    const bool valid = head < H;
    const int64_t g = g0 + j;
    const int64_t lo = max((int64_t)kGroup * g, rank * L);
    const int64_t hi = min((int64_t)kGroup * g + kGroup, rank * L + L);
    // Rows of the amax: [lo, amax_hi).  Rows of the min/max: [lo, min(hi, used)), which is
    // either the same range or empty (a group wholly in the zero tail), so one pass over
    // the amax rows serves both.
    const int64_t amax_hi =
        (p.used < p.S && g == (p.used - 1) / kGroup) ? min(hi, p.used) : hi;
    const int nrow = (int)(amax_hi - lo);           // may be <= 0
    const bool mm_live = min(hi, p.used) > lo;
    const bool want_amax = amax_out != nullptr;
    const bool want_mm = mm_out != nullptr && (j == 0 || j == n - 1);

    uint4 mraw = make_uint4(0, 0, 0, 0);
    if (p.mean[tensor] != nullptr && valid)
        mraw = load16(p.mean[tensor] + (b * H + head) * D + dv * 8);

    // Raw order statistics of this thread's rows lo + rl + 8i, i < 8, per channel: no
    // conversion or subtraction per element (the amax follows from the extremes below).
    // Rows past the range are replaced by its last row, which leaves every extreme as it
    // is and keeps the loop free of per-row branches.
    const uint16_t* xr =
        x + blockIdx.z * p.x_rank_stride + ((b * L + lo - rank * L) * H + head) * D + dv * 8;
    const bool mine = valid && rl < nrow;           // this thread has at least one row
    Order16 ord[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) ord[w].reset();
    if (mine) {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = load16<NT>(xr + (int64_t)min(rl + 8 * i, nrow - 1) * H * D);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ord[0].add(v[i].x);
            ord[1].add(v[i].y);
            ord[2].add(v[i].z);
            ord[3].add(v[i].w);
        }
    }

    // Per channel: the extremes as binary32 (zeros canonicalised to +0), then
    //   max over rows of |RN(x - m)| = max(RN(max x - m), RN(m - min x))
    // because RN(. - m) is non-decreasing and RN(-z) = -RN(z).
    float mn[8], mx[8], m[8];
    decode8<DT>(mraw, m);
    decode8<DT>(make_uint4(ord[0].min_bits(), ord[1].min_bits(), ord[2].min_bits(),
                           ord[3].min_bits()), mn);
    decode8<DT>(make_uint4(ord[0].max_bits(), ord[1].max_bits(), ord[2].max_bits(),
                           ord[3].max_bits()), mx);
    float acc = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn[e] = mine ? mn[e] + 0.0f : __builtin_inff();     // -0 -> +0
        mx[e] = mine ? mx[e] + 0.0f : -__builtin_inff();
        acc = fmaxf(acc, fmaxf(mx[e] - m[e], m[e] - mn[e]));
    }

    __shared__ float red_amax[4][HB];
    __shared__ float red_mn[4][32][8];
    __shared__ float red_mx[4][32][8];
    const int wave = tid >> 6, lane = tid & 63;
    if (want_amax) {
        // lanes sharing a head differ in the low log2(VPH) bits and in bit 5 (row lane)
        acc = wave_max_xor<(VPH - 1) | 32>(acc);
        if (lane < 32 && dv == 0) red_amax[wave][hib] = acc;
    }
    if (want_mm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            mn[e] = wave_min_xor<32>(mn[e]);
            mx[e] = wave_max_xor<32>(mx[e]);
        }
        if (lane < 32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                red_mn[wave][c][e] = mn[e];
                red_mx[wave][c][e] = mx[e];
            }
        }
    }
    __syncthreads();
    if (want_amax && tid < HB && (int64_t)hb * HB + tid < H) {
        float a = fmaxf(fmaxf(red_amax[0][tid], red_amax[1][tid]),
                        fmaxf(red_amax[2][tid], red_amax[3][tid]));
        amax_out[(b * H + hb * HB + tid) * p.slots + j] = fmaxf(kFloor, a);
    }
    if (want_mm && tid < 32 && valid) {
        float rmn[8], rmx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            rmn[e] = mm_live ? fminf(fminf(red_mn[0][c][e], red_mn[1][c][e]),
                                     fminf(red_mn[2][c][e], red_mn[3][c][e]))
                             : __builtin_inff();
            rmx[e] = mm_live ? fmaxf(fmaxf(red_mx[0][c][e], red_mx[1][c][e]),
                                     fmaxf(red_mx[2][c][e], red_mx[3][c][e]))
                             : -__builtin_inff();
        }
        for (int e2 = 0; e2 < 2; ++e2) {
            if ((e2 == 0 && j != 0) || (e2 == 1 && j != n - 1)) continue;
            float* o = mm_out + ((b * H + head) * 2 + e2) * 2 * D + dv * 8;
            float4* omn = reinterpret_cast<float4*>(o);
            float4* omx = reinterpret_cast<float4*>(o + D);
            omn[0] = make_float4(rmn[0], rmn[1], rmn[2], rmn[3]);
            omn[1] = make_float4(rmn[4], rmn[5], rmn[6], rmn[7]);
            omx[0] = make_float4(rmx[0], rmx[1], rmx[2], rmx[3]);
            omx[1] = make_float4(rmx[4], rmx[5], rmx[6], rmx[7]);
        }
    }
}

template <int DT, int D>
hipError_t launch_t(const StatsLaunch& a, hipStream_t stream) {
    StatsParams p;
    for (int t = 0; t < 2; ++t) {
        p.x[t] = a.x[t];
        p.mean[t] = a.mean[t];
        p.amax[t] = a.amax[t];
        p.minmax[t] = a.minmax[t];
    }
    p.x_rank_stride = a.x_rank_stride;
    p.amax_rank_stride = a.amax_rank_stride;
    p.minmax_rank_stride = a.minmax_rank_stride;
    p.L = a.L;
    p.H = a.H;
    p.S = a.P * a.L;
    p.used = a.used;
    p.slots = slots_of(a.L);
    p.rank0 = a.rank0;
    constexpr int HB = 256 / D;
    p.nhb = (int)((a.H + HB - 1) / HB);
    const bool any_amax = a.amax[0] != nullptr || a.amax[1] != nullptr;
    p.boundary_only = any_amax ? 0 : 1;
    p.grid_slots = any_amax ? (int)p.slots : 2;
    dim3 grid((unsigned)(a.B * p.grid_slots * p.nhb), a.x[1] ? 2 : 1, (unsigned)a.nranks);
    const int64_t streamed = (a.x[1] ? 2 : 1) * a.nranks * a.B * a.L * a.H * D * 2;
    if (streamed > kResidentBytes)
        hipLaunchKernelGGL((stats_kernel<DT, D, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((stats_kernel<DT, D, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stats(const StatsLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64>(a, stream)
                                           : launch_t<kBF16, 128>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64>(a, stream) : launch_t<kFP16, 128>(a, stream);
}

}  // namespace ulp
