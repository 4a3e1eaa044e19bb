// kmean.hip -- the global K mean over the live rows of a Ulysses group (gfx950).
//
// The k_grouped_amax and derive_k_boundary_amax pages take k_mean_global as an input: a
// [B, H, D] mean of K over the global sequence, already rounded to the input dtype.  On one
// GPU that holds the whole group it is formed here from the stacked shards [P, B, L, H, D]:
// the sum over live rows [0, used) in binary64, divided by used in binary64, rounded to
// binary32 (returned) and from there to the dtype (returned when asked for).
//
// Deterministic two-stage reduction, its order fixed by the shape alone:
//   * partial: one 256-thread workgroup per (column block of 512 values, chunk of `rows`
//     rows, b).  Every wave covers the block's 512 values (a lane owns one 16-byte vector,
//     8 values) over a quarter of the chunk's rows, 8 row loads in flight, 8 binary64 sums
//     per lane; the four waves' sums are added in wave order through LDS and written to the
//     caller's workspace [chunks, B, H*D] binary64.
//   * finalize: one workgroup per 64 (b, value) pairs; each wave adds a contiguous quarter
//     of the chunks in chunk order, the quarters are added in order, then divided and
//     rounded.
// The chunk height is chosen from the shape so that the partial pass has about 2048
// workgroups.  A binary64 sum of 16-bit inputs over < 2^31 rows carries a relative error far
// below the 1e-6 the mean is held to; where every partial sum is exact (inputs whose
// exponents span less than ~2^20 at these row counts) the result equals the sequential
// binary64 definition bit for bit.
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr int kColsPerBlock = 64 * 8;     // one wave-wide row segment
constexpr int kMinRows = 32, kMaxRows = 512;
constexpr int64_t kTargetBlocks = 512;

struct KMeanParams {
    const uint16_t* k;
    double* partial;
    float* mean_f32;
    uint16_t* mean_dt;
    int64_t B, L, HD, used, rows, chunks;
};

template <int DT, bool NT>
__global__ __launch_bounds__(kThreads) void kmean_partial_kernel(KMeanParams p) {
    __shared__ double red[kWaves - 1][8][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * kColsPerBlock + lane * 8;
    const int64_t chunk = blockIdx.y, b = blockIdx.z;
    const int64_t per_wave = p.rows / kWaves;   // a multiple of 8
    const int64_t t0 = chunk * p.rows + wave * per_wave;
    const int64_t t1 = min(t0 + per_wave, p.used);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    if (col < p.HD && t0 < t1) {
        int64_t r = t0 / p.L, l = t0 - r * p.L;   // shard and local row of global row t
        const uint16_t* kc = p.k + col;
        for (int64_t t = t0; t < t1; t += 8) {
            uint4 v[8];
            if (l + 8 <= p.L && t + 8 <= t1) {
                // the whole batch in one shard and in the range (the common case; the
                // test is the same for every lane): consecutive rows, one stride apart
                const uint16_t* rp = kc + ((r * p.B + b) * p.L + l) * p.HD;
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = load16<NT>(rp + i * p.HD);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float f[8];
                    decode8<DT>(v[i], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    int64_t ri = r, li = l + i;
                    while (li >= p.L) {    // 8 rows span at most 8 shard boundaries
                        li -= p.L;
                        ++ri;
                    }
                    v[i] = t + i < t1 ? load16<NT>(kc + ((ri * p.B + b) * p.L + li) * p.HD)
                                      : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (t + i >= t1) break;
                    float f[8];
                    decode8<DT>(v[i], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
                }
            }
            l += 8;
            while (l >= p.L) {
                l -= p.L;
                ++r;
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave - 1][e][lane] = acc[e];
    }
    __syncthreads();
    if (wave == 0 && col < p.HD) {
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += red[w][e][lane];
        double* out = p.partial + (chunk * p.B + b) * p.HD + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = acc[e];
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

template <int DT>
__global__ __launch_bounds__(kThreads) void kmean_finalize_kernel(KMeanParams p) {
    __shared__ double red[kWaves - 1][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n = p.B * p.HD;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;            // (b, value)
    const int64_t q = (p.chunks + kWaves - 1) / kWaves;
    const int64_t c0 = wave * q, c1 = min(c0 + q, p.chunks);
    double sum = 0.0;
    if (i < n) {
        const double* src = p.partial + i;
        int64_t c = c0;
        for (; c + 8 <= c1; c += 8) {
            double v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = src[(c + j) * n];
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += v[j];
        }
        for (; c < c1; ++c) sum += src[c * n];
    }
    if (wave > 0) red[wave - 1][lane] = sum;
    __syncthreads();
    if (wave == 0 && i < n) {
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w) sum += red[w][lane];
        const float m = (float)(sum / (double)p.used);
        p.mean_f32[i] = m;
        if (p.mean_dt) p.mean_dt[i] = round_to_dtype<DT>(m);
    }
}

int64_t col_blocks(int64_t HD) { return (HD + kColsPerBlock - 1) / kColsPerBlock; }

template <int DT>
hipError_t launch_t(const KMeanLaunch& a, hipStream_t stream) {
    KMeanParams p;
    p.k = a.k;
    p.partial = a.workspace;
    p.mean_f32 = a.mean_f32;
    p.mean_dt = a.mean_dtype;
    p.B = a.B;
    p.L = a.L;
    p.HD = a.H * a.D;
    p.used = a.used;
    p.rows = kmean_rows(a.B, a.H, a.D, a.used);
    p.chunks = (a.used + p.rows - 1) / p.rows;
    dim3 g1((unsigned)col_blocks(p.HD), (unsigned)p.chunks, (unsigned)a.B);
    const bool nt = 2 * a.B * a.used * p.HD > kResidentBytes;
    if (nt)
        hipLaunchKernelGGL((kmean_partial_kernel<DT, true>), g1, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((kmean_partial_kernel<DT, false>), g1, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2((unsigned)((a.B * p.HD + 63) / 64));
    hipLaunchKernelGGL((kmean_finalize_kernel<DT>), g2, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int64_t kmean_rows(int64_t B, int64_t H, int64_t D, int64_t used) {
    const int64_t base = B * col_blocks(H * D);
    int64_t r = kMinRows;
    while (r < kMaxRows && base * ((used + 2 * r - 1) / (2 * r)) >= kTargetBlocks) r *= 2;
    return r;
}

int64_t kmean_chunks(int64_t B, int64_t H, int64_t D, int64_t used) {
    const int64_t r = kmean_rows(B, H, D, used);
    return (used + r - 1) / r;
}

hipError_t launch_kmean(const KMeanLaunch& a, hipStream_t stream) {
    return a.dtype == kBF16 ? launch_t<kBF16>(a, stream) : launch_t<kFP16>(a, stream);
}

}  // namespace ulp
