// kstats.hip -- K statistics and the global K mean from one read of K (gfx950).
//
// k_grouped_amax (description) centers K by k_mean_global before the amax, so the amax pass
// needs the mean first, and forming the mean is itself a pass over K.  Both come out of one
// pass here, because the centered amax of a group is a function of the group's per-channel
// raw minimum and maximum: RN is monotone and RN(-x) = -RN(x), so over the rows of a group,
//   max_rows |RN(k - m)| = max(RN(max_rows k - m), RN(m - min_rows k))      (per channel)
// which is the same identity derive_k_boundary_amax (description) rests on.  The pass records
// per (rank, b, head, slot, channel) the raw min / max over the rows the amax runs on (as
// the 16-bit inputs themselves) and the binary64 sum over the live rows; then
//   * kmean_from_sums adds the sums in (rank, slot) order (16 contiguous parts, then the
//     parts in order), divides by used in binary64 and rounds to binary32 and to the dtype
//     (the same definition as ulp_k_mean);
//   * kamax_from_minmax forms every slot's amax from the min / max and the dtype-rounded
//     mean, bit-identical to the direct pass;
// and the boundary min / max of every rank are written by the pass itself.
#include "order16.h"
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

struct KStatsParams {
    const uint16_t* k;       // stacked [P, B, L, H, D]
    uint16_t* mm;            // [P, B, H, slots, 2, D] raw min (0) / max (1) over amax rows
    double* sum;             // [P, B, H, slots, D] binary64 sums over live rows
    float* minmax;           // [P, B, H, 2, 2, D] boundary min / max (live rows)
    float* amax;             // [P, B, H, slots]
    float* mean_f32;         // [B, H, D]
    uint16_t* mean_dt;       // [B, H, D]
    int64_t B, L, H, S, used, slots;
    int P, nhb;
};

// One 256-thread workgroup per (rank, b, slot, head block), as the statistics kernel: 64
// rows x 32 sixteen-byte vectors, thread (row lane rl, vector c) reading rows rl + 8i.
// The raw extremes are kept as Order16 (packed integer operations, no conversion); the
// sums take the binary64 value of every live element.  The eight row lanes are combined
// through LDS and the results written by all 256 threads, one (vector, channel) each.
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
    // The amax runs over every row of the group except past `used` in the one partial live
    // group (k_grouped_amax, used_sequence); the sums and the boundary min/max over the live
    // rows, which are the same rows or none (a group wholly in the zero tail).
    const int64_t amax_hi =
        (p.used < p.S && g == (p.used - 1) / kGroup) ? min(hi, p.used) : hi;
    const int nrow = (int)(amax_hi - lo);            // may be <= 0
    const bool live = min(hi, p.used) > lo;

    const uint16_t* xr = p.k + (((rank * p.B + b) * L + lo - rank * L) * H + head) * D + dv * 8;
    Order16 ord[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) ord[w].reset();
    // Sums start at -0, the identity of IEEE addition (x + -0 = x for every x, +0 included),
    // so the first addend costs nothing; the mean's sum over slots starts at +0.
    double sm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[e] = -0.0;
    if (valid && rl < nrow) {
        // rows past the range repeat its last row: harmless for the extremes, masked out
        // of the sums
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
        if (nrow == kGroup) {                        // a whole live group: no masking
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float f[8];
                decode8<DT>(v[i], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) sm[e] += (double)f[e];
            }
        } else if (live) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float f[8];
                decode8<DT>(v[i], f);
                const bool in = rl + 8 * i < nrow;
#pragma unroll
                for (int e = 0; e < 8; ++e) sm[e] += (double)(in ? f[e] : -0.0f);
            }
        }
    }

    // Row lanes: bit 5 of the lane inside a wave (v_permlane32_swap hands each lane the
    // value of its partner 32 lanes away; merging and adding are symmetric, so both halves
    // end with the same bits), then the four waves through LDS.
    __shared__ Order16 red_ord[4][32][4];
    __shared__ double red_sm[4][32][8];
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(ord[w].smax, ord[w].smax, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(ord[w].umin, ord[w].umin, false, false);
        const auto s2 = __builtin_amdgcn_permlane32_swap(ord[w].umax, ord[w].umax, false, false);
        ord[w] = merge(Order16{s0[0], s1[0], s2[0]}, Order16{s0[1], s1[1], s2[1]});
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint64_t u = __builtin_bit_cast(uint64_t, sm[e]);
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                         false, false);
        sm[e] = __builtin_bit_cast(double, (uint64_t)lo[0] | ((uint64_t)hi[0] << 32)) +
                __builtin_bit_cast(double, (uint64_t)lo[1] | ((uint64_t)hi[1] << 32));
    }
    if (lane < 32) {
#pragma unroll
        for (int w = 0; w < 4; ++w) red_ord[wave][c][w] = ord[w];
#pragma unroll
        for (int e = 0; e < 8; ++e) red_sm[wave][c][e] = sm[e];
    }
    __syncthreads();

    // Thread (vector c2, channel pair or channel e2): the four waves in order.
    const int c2 = tid >> 3, e2 = tid & 7;
    const int hib2 = c2 / VPH, dv2 = c2 % VPH;
    const int64_t head2 = (int64_t)hb * HB + hib2;
    if (head2 >= H) return;
    const int64_t rbh = (rank * p.B + b) * H + head2;
    const double s4 =
        ((red_sm[0][c2][e2] + red_sm[1][c2][e2]) + red_sm[2][c2][e2]) + red_sm[3][c2][e2];
    p.sum[(rbh * p.slots + j) * D + dv2 * 8 + e2] = s4;
    if (e2 >= 4) return;
    const int w2 = e2;                              // channels 2 w2, 2 w2 + 1 of vector c2
    const Order16 o4 = merge(merge(red_ord[0][c2][w2], red_ord[1][c2][w2]),
                             merge(red_ord[2][c2][w2], red_ord[3][c2][w2]));
    const uint32_t mnb = o4.min_bits(), mxb = o4.max_bits();
    uint16_t* o = p.mm + ((rbh * p.slots + j) * 2) * D + dv2 * 8 + 2 * w2;
    *reinterpret_cast<uint32_t*>(o) = mnb;
    *reinterpret_cast<uint32_t*>(o + D) = mxb;
    // Boundary min / max over live rows, zeros as +0; a group with no live row gives
    // (+inf, -inf).
    if (j != 0 && j != n - 1) return;
    float mn0, mn1, mx0, mx1;
    decode2<DT>(mnb, mn0, mn1);
    decode2<DT>(mxb, mx0, mx1);
    const float inf = __builtin_inff();
    for (int eb = 0; eb < 2; ++eb) {
        if ((eb == 0 && j != 0) || (eb == 1 && j != n - 1)) continue;
        float* ob = p.minmax + (rbh * 2 + eb) * 2 * D + dv2 * 8 + 2 * w2;
        *reinterpret_cast<float2*>(ob) =
            live ? make_float2(mn0 + 0.0f, mn1 + 0.0f) : make_float2(inf, inf);
        *reinterpret_cast<float2*>(ob + D) =
            live ? make_float2(mx0 + 0.0f, mx1 + 0.0f) : make_float2(-inf, -inf);
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
// workgroup covers 16 consecutive (b, head, channel) values (128-byte loads) and splits the
// (rank, slot) sequence into 16 contiguous parts, four per wave; each part is added in
// order with 8 loads in flight, then the parts in order.
constexpr int kSumParts = 16;

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void kmean_from_sums_kernel(KStatsParams p) {
    __shared__ double red[kSumParts][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int dl = lane & 15, part = wave * 4 + (lane >> 4);
    const int64_t i = (int64_t)blockIdx.x * 16 + dl;             // (b, head, d)
    const int64_t nv = p.B * p.H * D;
    const int64_t d = i % D, bh = i / D;
    int64_t total = 0;
    for (int r = 0; r < p.P; ++r) total += last_group(r, p.L) - first_group(r, p.L) + 1;
    const int64_t q0 = total * part / kSumParts, q1 = total * (part + 1) / kSumParts;
    double sum = 0.0;
    if (i < nv && q0 < q1) {
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
    red[part][dl] = sum;
    __syncthreads();
    if (threadIdx.x >= 16 || i >= nv) return;
    sum = red[0][dl];
#pragma unroll
    for (int k = 1; k < kSumParts; ++k) sum += red[k][dl];
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
        const uint16_t* o = p.mm + (rbh * p.slots + j) * 2 * D;
        const uint16_t* mp = p.mean_dt + bh * D;
#pragma unroll
        for (int d = lane; d < D; d += 64) {
            const float m = decode1<DT>(mp[d]);
            a = fmaxf(a, fmaxf(decode1<DT>(o[D + d]) - m, m - decode1<DT>(o[d])));
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
    const dim3 g2((unsigned)((a.B * a.H * D + 15) / 16));
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
