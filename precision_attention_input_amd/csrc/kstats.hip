// kstats.hip -- K statistics and the global K mean from one read of K (gfx950).
//
// k_grouped_amax (description) centers K by k_mean_global before the amax, so the amax pass
// needs the mean first, and forming the mean is itself a pass over K.  Both come out of one
// pass here, because the centered amax of a group is a function of the group's per-channel
// raw minimum and maximum: RN is monotone and RN(-x) = -RN(x), so over the rows of a group,
//   max_rows |RN(k - m)| = max(RN(max_rows k - m), RN(m - min_rows k))      (per channel)
// which is the same identity derive_k_boundary_amax (description) rests on.  The pass records
// per (rank, b, head, slot, channel) the raw min / max over the rows the amax runs on and the
// binary64 sum over the live rows; then
//   * kmean_from_sums adds the sums in (rank, slot) order (four contiguous quarters, then the
//     quarters in order), divides by used in binary64 and rounds to binary32 and to the
//     dtype (the same definition as ulp_k_mean);
//   * kamax_from_minmax forms every slot's amax from the min / max and the dtype-rounded
//     mean, bit-identical to the direct pass;
// and the boundary min / max of every rank are written by the pass itself.
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

struct KStatsParams {
    const uint16_t* k;       // stacked [P, B, L, H, D]
    float* mm;               // [P, B, H, slots, 2, D] raw min (0) / max (1) over amax rows
    double* sum;             // [P, B, H, slots, D] binary64 sums over live rows
    float* minmax;           // [P, B, H, 2, 2, D] boundary min / max (live rows)
    float* amax;             // [P, B, H, slots]
    float* mean_f32;         // [B, H, D]
    uint16_t* mean_dt;       // [B, H, D]
    int64_t B, L, H, S, used, slots;
    int P, nhb;
};

template <int DT, int D, bool NT>
__global__ __launch_bounds__(kThreads) void kstats_kernel(KStatsParams p) {
    constexpr int VPH = D / 8;       // 16-byte vectors per head row
    constexpr int HB = 256 / D;      // heads per workgroup: 32 vectors per row
    const int64_t L = p.L, H = p.H;
    const int64_t rank = blockIdx.z;
    int bid = blockIdx.x;
    const int hb = bid % p.nhb;
    bid /= p.nhb;
    const int64_t j = bid % p.slots;
    const int64_t b = bid / p.slots;
    const int64_t g0 = first_group(rank, L);
    const int64_t n = last_group(rank, L) - g0 + 1;
    if (j >= n) return;              // a slot this rank never touches: nothing recorded

    const int tid = threadIdx.x;
    const int c = tid & 31, rl = tid >> 5;
    const int hib = c / VPH, dv = c % VPH;
    const int64_t head = (int64_t)hb * HB + hib;
    const bool valid = head < H;
    const int64_t g = g0 + j;
    const int64_t lo = max((int64_t)kGroup * g, rank * L);
    const int64_t hi = min((int64_t)kGroup * g + kGroup, rank * L + L);
    // the amax runs over every row of the group except past `used` in the one partial live
    // group (k_grouped_amax, used_sequence); the sums over live rows
    const int64_t amax_hi =
        (p.used < p.S && g == (p.used - 1) / kGroup) ? min(hi, p.used) : hi;
    const int64_t live_hi = min(hi, p.used);

    const uint16_t* xb = p.k + ((rank * p.B + b) * L * H + head) * D + dv * 8;
    float mn[8], mx[8];
    double sm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn[e] = __builtin_inff();
        mx[e] = -__builtin_inff();
        sm[e] = 0.0;
    }
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t s = lo + rl + 8 * i;
        v[i] = (valid && s < hi) ? load16<NT>(xb + (s - rank * L) * H * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t s = lo + rl + 8 * i;
        if (!(valid && s < amax_hi)) continue;
        float f[8];
        decode8<DT>(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float cv = f[e] + 0.0f;   // -0 -> +0, every other value unchanged
            mn[e] = fminf(mn[e], cv);
            mx[e] = fmaxf(mx[e], cv);
            if (s < live_hi) sm[e] += (double)f[e];
        }
    }

    // Reduce over the 8 row lanes: bit 5 of the lane inside a wave, then the 4 waves in
    // order through LDS.
    __shared__ float red_mn[4][32][8];
    __shared__ float red_mx[4][32][8];
    __shared__ double red_sm[4][32][8];
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn[e] = wave_min_xor<32>(mn[e]);
        mx[e] = wave_max_xor<32>(mx[e]);
        const double other = __shfl_xor(sm[e], 32, 64);
        sm[e] = lane < 32 ? sm[e] + other : other + sm[e];
    }
    if (lane < 32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red_mn[wave][c][e] = mn[e];
            red_mx[wave][c][e] = mx[e];
            red_sm[wave][c][e] = sm[e];
        }
    }
    __syncthreads();
    if (tid >= 32 || !valid) return;
    float rmn[8], rmx[8];
    double rsm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        rmn[e] = fminf(fminf(red_mn[0][c][e], red_mn[1][c][e]),
                       fminf(red_mn[2][c][e], red_mn[3][c][e]));
        rmx[e] = fmaxf(fmaxf(red_mx[0][c][e], red_mx[1][c][e]),
                       fmaxf(red_mx[2][c][e], red_mx[3][c][e]));
        rsm[e] = ((red_sm[0][c][e] + red_sm[1][c][e]) + red_sm[2][c][e]) + red_sm[3][c][e];
    }
    const int64_t rbh = (rank * p.B + b) * H + head;
    float* o = p.mm + ((rbh * p.slots + j) * 2) * D + dv * 8;
    double* os = p.sum + (rbh * p.slots + j) * D + dv * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] = rmn[e];
        o[D + e] = rmx[e];
        os[e] = rsm[e];
    }
    // Boundary min / max over live rows: the same values, except that a fully padded group
    // has no live row.
    const bool empty = lo >= p.used;
    for (int e2 = 0; e2 < 2; ++e2) {
        if ((e2 == 0 && j != 0) || (e2 == 1 && j != n - 1)) continue;
        float* ob = p.minmax + (rbh * 2 + e2) * 2 * D + dv * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ob[e] = empty ? __builtin_inff() : rmn[e];
            ob[D + e] = empty ? -__builtin_inff() : rmx[e];
        }
    }
}

template <int DT>
__device__ __forceinline__ uint16_t round_to_dtype(float m) {
    if constexpr (DT == kBF16) {
        const uint32_t u = __float_as_uint(m);
        return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // nearest even
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)m);            // v_cvt_f16_f32, RNE
    }
}

// The sums of every rank's touched slots in (rank, slot) order, per (b, head, channel): a
// workgroup covers 64 consecutive (b, head, channel) values; wave w adds the w-th quarter
// of the (rank, slot) sequence in order, 8 loads in flight, and the quarters are added in
// order.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void kmean_from_sums_kernel(KStatsParams p) {
    __shared__ double red[3][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;            // (b, head, d)
    const int64_t nv = p.B * p.H * D;
    const int64_t d = i % D, bh = i / D;
    int64_t total = 0;
    for (int r = 0; r < p.P; ++r) total += last_group(r, p.L) - first_group(r, p.L) + 1;
    const int64_t q0 = total * wave / 4, q1 = total * (wave + 1) / 4;
    double sum = 0.0;
    if (i < nv) {
        // walk (rank, slot) pairs from flat index q0
        int r = 0;
        int64_t base = 0, n = last_group(0, p.L) - first_group(0, p.L) + 1;
        while (q0 >= base + n) {
            base += n;
            ++r;
            n = last_group(r, p.L) - first_group(r, p.L) + 1;
        }
        int64_t jj = q0 - base;
        int64_t q = q0;
        while (q < q1) {
            const double* s = p.sum + ((int64_t)r * p.B * p.H + bh) * p.slots * D + d;
            const int64_t m = min(n - jj, q1 - q);     // slots of this rank in the range
            int64_t t = 0;
            for (; t + 8 <= m; t += 8) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = s[(jj + t + u) * D];
#pragma unroll
                for (int u = 0; u < 8; ++u) sum += v[u];
            }
            for (; t < m; ++t) sum += s[(jj + t) * D];
            q += m;
            ++r;
            jj = 0;
            if (r < p.P) n = last_group(r, p.L) - first_group(r, p.L) + 1;
        }
    }
    if (wave > 0) red[wave - 1][lane] = sum;
    __syncthreads();
    if (wave != 0 || i >= nv) return;
    sum = ((sum + red[0][lane]) + red[1][lane]) + red[2][lane];
    const float mf = (float)(sum / (double)p.used);
    p.mean_f32[i] = mf;
    p.mean_dt[i] = round_to_dtype<DT>(mf);
}

// One wave per (rank, b, head, slot): max over channels of max(RN(mx - m), RN(m - mn)),
// floored; slots the rank does not touch hold the floor.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void kamax_from_minmax_kernel(KStatsParams p) {
    const int64_t item = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= (int64_t)p.P * p.B * p.H * p.slots) return;
    const int64_t j = item % p.slots, rbh = item / p.slots;
    const int64_t bh = rbh % (p.B * p.H);
    const int64_t r = rbh / (p.B * p.H);
    const int64_t n = last_group(r, p.L) - first_group(r, p.L) + 1;
    float a = -__builtin_inff();
    if (j < n) {
        const float* o = p.mm + (rbh * p.slots + j) * 2 * D;
        const uint16_t* mp = p.mean_dt + bh * D;
#pragma unroll
        for (int d = lane; d < D; d += 64) {
            const float m = decode1<DT>(mp[d]);
            a = fmaxf(a, fmaxf(o[D + d] - m, m - o[d]));
        }
    }
    a = wave_max_xor<63>(a);
    if (lane == 0) p.amax[rbh * p.slots + j] = j < n ? fmaxf(kFloor, a) : kFloor;
}

template <int DT, int D>
hipError_t launch_t(const KStatsLaunch& a, hipStream_t stream) {
    KStatsParams p;
    p.k = a.k;
    p.mm = a.mm;
    p.sum = a.sum;
    p.minmax = a.minmax;
    p.amax = a.amax;
    p.mean_f32 = a.mean_f32;
    p.mean_dt = a.mean_dtype;
    p.B = a.B;
    p.L = a.L;
    p.H = a.H;
    p.S = a.P * a.L;
    p.used = a.used;
    p.slots = slots_of(a.L);
    p.P = (int)a.P;
    constexpr int HB = 256 / D;
    p.nhb = (int)((a.H + HB - 1) / HB);
    const dim3 g1((unsigned)(a.B * p.slots * p.nhb), 1, (unsigned)a.P);
    const bool nt = a.P * a.B * a.L * a.H * D * 2 > kResidentBytes;
    if (nt)
        hipLaunchKernelGGL((kstats_kernel<DT, D, true>), g1, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((kstats_kernel<DT, D, false>), g1, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((a.B * a.H * D + 63) / 64));
    hipLaunchKernelGGL((kmean_from_sums_kernel<DT, D>), g2, dim3(kThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t waves = a.P * a.B * a.H * p.slots;
    const dim3 g3((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)));
    hipLaunchKernelGGL((kamax_from_minmax_kernel<DT, D>), g3, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kstats(const KStatsLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64>(a, stream)
                                           : launch_t<kBF16, 128>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64>(a, stream) : launch_t<kFP16, 128>(a, stream);
}

}  // namespace ulp
