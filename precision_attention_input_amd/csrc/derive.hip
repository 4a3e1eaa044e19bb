// derive.hip -- cross-rank boundary-group amax from gathered raw min/max (gfx950).
//
// flashinfer.comm._ulysses_lowp.derive_k_boundary_amax (description): for each of a rank's
// first and last touched groups g, the slot becomes the max over every rank r touching g of
//   contrib(r, g) = max(1e-7, max_d max(RN(maxK[r,g,d] - m[d]), RN(m[d] - minK[r,g,d]))).
// RN subtraction is monotone, so this equals r's direct |K - m| amax over its slice of g;
// every rank evaluates the same exact operations on the same gathered data and so ends
// with the same bits.  A padding-only slice carries (+inf, -inf) and contributes exactly
// the floor.
//
// One wave per (rank, tensor, b, head, boundary); lanes cover the channels, a wave-wide
// max tree reduces them.
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

struct DeriveParams {
    float* amax[2];
    const float* minmax[2];
    const uint16_t* mean[2];
    int64_t amax_rank_stride;
    int64_t B, H, L, P, slots;
    int rank0;
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void derive_kernel(DeriveParams p) {
    constexpr int PER_LANE = D / 64;
    const int tensor = blockIdx.y;
    float* amax = p.amax[tensor];
    if (amax == nullptr) return;
    const int64_t rank = p.rank0 + blockIdx.z;
    amax += blockIdx.z * p.amax_rank_stride;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, head, e)
    if (item >= p.B * p.H * 2) return;
    const int e = (int)(item & 1);
    const int64_t bh = item >> 1;
    const int64_t b = bh / p.H, head = bh % p.H;
    const int64_t L = p.L;
    const int64_t g0 = first_group(rank, L), g1 = last_group(rank, L);
    if (e == 1 && g1 == g0) return;    // one touched group: the e = 0 wave writes it
    const int64_t g = e == 0 ? g0 : g1;

    float m[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
        m[i] = p.mean[tensor] ? decode1<DT>(p.mean[tensor][(b * p.H + head) * D + lane + 64 * i])
                              : 0.0f;
    const float* mm = p.minmax[tensor];
    float best = -__builtin_inff();
    for (int64_t r = 0; r < p.P; ++r) {
        const bool touches = r * L < kGroup * g + kGroup && kGroup * g < r * L + L;
        if (!touches) continue;
        const int er = (g == first_group(r, L)) ? 0 : 1;
        const float* base = mm + ((((r * p.B + b) * p.H + head) * 2 + er) * 2) * D;
        float cmax = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const float mn = base[lane + 64 * i];
            const float mx = base[D + lane + 64 * i];
            cmax = fmaxf(cmax, fmaxf(mx - m[i], m[i] - mn));
        }
        cmax = wave_max_xor<63>(cmax);
        best = fmaxf(best, fmaxf(kFloor, cmax));
    }
    if (lane == 0) amax[(b * p.H + head) * p.slots + (g - g0)] = best;
}

template <int DT, int D>
hipError_t launch_t(const DeriveLaunch& a, hipStream_t stream) {
    DeriveParams p;
    for (int t = 0; t < 2; ++t) {
        p.amax[t] = a.amax[t];
        p.minmax[t] = a.minmax[t];
        p.mean[t] = a.mean[t];
    }
    p.amax_rank_stride = a.amax_rank_stride;
    p.B = a.B;
    p.H = a.H;
    p.L = a.L;
    p.P = a.P;
    p.slots = slots_of(a.L);
    p.rank0 = a.rank0;
    const int64_t items = a.B * a.H * 2;
    dim3 grid((unsigned)((items + 3) / 4), a.amax[1] ? 2 : 1, (unsigned)a.nranks);
    hipLaunchKernelGGL((derive_kernel<DT, D>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_derive(const DeriveLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64>(a, stream)
                                           : launch_t<kBF16, 128>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64>(a, stream) : launch_t<kFP16, 128>(a, stream);
}

}  // namespace ulp
