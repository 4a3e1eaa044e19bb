// pack.hip -- quantize one rank's shard into per-destination chunks (gfx950).
//
// The pack step the k_grouped_amax page (description) refers to: per global 64-row group a
// scale = RN(amax / 127); every element becomes
//   q8 = clamp(rint(RN(fp32(q) / q_scale)), -127, 127)
//   k8 = clamp(rint(RN(RN(fp32(k) - fp32(mean)) / k_scale)), -127, 127)
//   v8 = E4M3FN(fp32(v)) (nearest even, saturating)
// and lands in the chunk of the destination owning its head (unpack_for_sage Parameters:
// local_heads = H / world_size, contiguous per destination).  Chunk sections: q8, k8, v8
// [B, L, h, D] bytes, then q_scale, k_scale [B, h, slots] fp32, each 256-byte aligned.
//
// Work decomposition: one 256-thread workgroup per (rank, b, slot, block of 512 / D heads);
// a row of the block is 512 elements = 32 threads x 16 elements, so 8 rows are in flight and
// each thread walks the group's rows with stride 8.  Every thread loads 2 x 16 bytes of each
// of Q, K and V per row and stores 16 bytes of each code tensor -- fully coalesced on both
// sides.  The per-group scale and its reciprocal are computed once per thread.
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

struct PackParams {
    const uint16_t *q, *k, *v, *mean;
    const float *q_amax, *k_amax;
    uint8_t* send;
    int64_t dest_stride, x_rank_stride, amax_rank_stride, send_rank_stride;
    int64_t B, L, H, h, P, slots, sec, ssec;
    int rank0, nhb;
};

template <int DT>
__device__ __forceinline__ void decode16(const uint4& a, const uint4& b, float* f) {
    decode8<DT>(a, f);
    decode8<DT>(b, f + 8);
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p) {
    constexpr int VPH = D / 16;      // 16-element vectors per head row
    constexpr int HB = 512 / D;      // heads per workgroup
    const int64_t L = p.L, H = p.H, h = p.h;
    const int64_t rank = p.rank0 + blockIdx.z;
    uint8_t* send = p.send + blockIdx.z * p.send_rank_stride;
    int bid = blockIdx.x;
    const int hb = bid % p.nhb;
    bid /= p.nhb;
    const int64_t j = bid % p.slots;
    const int64_t b = bid / p.slots;
    const int tid = threadIdx.x;

    if (blockIdx.x == 0) {
        // Zero the padding bytes after each section of every destination chunk.
        const int64_t data = p.B * L * h * D;                       // bytes of q8/k8/v8 data
        const int64_t sdata = 4 * p.B * h * p.slots;                // bytes of scale data
        for (int64_t i = tid; i < p.P * 5 * 256; i += kThreads) {
            const int64_t dst = i / (5 * 256), sect = (i / 256) % 5, off = i % 256;
            const int64_t start = sect < 3 ? sect * p.sec + data
                                           : 3 * p.sec + (sect - 3) * p.ssec + sdata;
            const int64_t end = sect < 3 ? (sect + 1) * p.sec : 3 * p.sec + (sect - 2) * p.ssec;
            if (start + off < end) send[dst * p.dest_stride + start + off] = 0;
        }
    }

    const int c = tid & 31, rl = tid >> 5;
    const int hib = c / VPH, dv = c % VPH;
    const int64_t head = (int64_t)hb * HB + hib;
    if (head >= H) return;
    const int64_t dst = head / h, jl = head % h;
    uint8_t* chunk = send + dst * p.dest_stride;
    const float* qa = p.q_amax + blockIdx.z * p.amax_rank_stride;
    const float* ka = p.k_amax + blockIdx.z * p.amax_rank_stride;
    const QuantScale sq = make_scale(qa[(b * H + head) * p.slots + j]);
    const QuantScale sk = make_scale(ka[(b * H + head) * p.slots + j]);
    if (rl == 0 && dv == 0) {
        float* qs = reinterpret_cast<float*>(chunk + 3 * p.sec);
        float* ks = reinterpret_cast<float*>(chunk + 3 * p.sec + p.ssec);
        qs[(b * h + jl) * p.slots + j] = sq.s;
        ks[(b * h + jl) * p.slots + j] = sk.s;
    }
    const int64_t g0 = first_group(rank, L);
    const int64_t n = last_group(rank, L) - g0 + 1;
    if (j >= n) return;
    const int64_t g = g0 + j;
    const int64_t lo = max((int64_t)kGroup * g, rank * L) - rank * L;
    const int64_t hi = min((int64_t)kGroup * g + kGroup, rank * L + L) - rank * L;

    float m[16];
    {
        const uint16_t* mp = p.mean + (b * H + head) * D + dv * 16;
        decode16<DT>(load16(mp), load16(mp + 8), m);
    }
    const int64_t xoff0 = blockIdx.z * p.x_rank_stride + (b * L * H + head) * D + dv * 16;
    const int64_t ooff0 = (b * L * h + jl) * D + dv * 16;
    int8_t* q8 = reinterpret_cast<int8_t*>(chunk);
    int8_t* k8 = reinterpret_cast<int8_t*>(chunk + p.sec);
    uint8_t* v8 = chunk + 2 * p.sec;

    for (int64_t l = lo + rl; l < hi; l += 8) {
        const int64_t xo = xoff0 + l * H * D;
        const uint4 qa0 = load16(p.q + xo), qa1 = load16(p.q + xo + 8);
        const uint4 ka0 = load16(p.k + xo), ka1 = load16(p.k + xo + 8);
        const uint4 va0 = load16(p.v + xo), va1 = load16(p.v + xo + 8);
        float f[16], r[16];
        uint4 out;
        const int64_t oo = ooff0 + l * h * D;

        decode16<DT>(qa0, qa1, f);
        quantize_n<16>(f, sq, r);
        out.x = pack_i8x4(r[0], r[1], r[2], r[3]);
        out.y = pack_i8x4(r[4], r[5], r[6], r[7]);
        out.z = pack_i8x4(r[8], r[9], r[10], r[11]);
        out.w = pack_i8x4(r[12], r[13], r[14], r[15]);
        store16(q8 + oo, out);

        decode16<DT>(ka0, ka1, f);
#pragma unroll
        for (int e = 0; e < 16; ++e) f[e] = f[e] - m[e];
        quantize_n<16>(f, sk, r);
        out.x = pack_i8x4(r[0], r[1], r[2], r[3]);
        out.y = pack_i8x4(r[4], r[5], r[6], r[7]);
        out.z = pack_i8x4(r[8], r[9], r[10], r[11]);
        out.w = pack_i8x4(r[12], r[13], r[14], r[15]);
        store16(k8 + oo, out);

        decode16<DT>(va0, va1, f);
        out.x = e4m3x4(f[0], f[1], f[2], f[3]);
        out.y = e4m3x4(f[4], f[5], f[6], f[7]);
        out.z = e4m3x4(f[8], f[9], f[10], f[11]);
        out.w = e4m3x4(f[12], f[13], f[14], f[15]);
        store16(v8 + oo, out);
    }
}

template <int DT, int D>
hipError_t launch_t(const PackLaunch& a, hipStream_t stream) {
    PackParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.mean = a.mean;
    p.q_amax = a.q_amax;
    p.k_amax = a.k_amax;
    p.send = a.send;
    p.dest_stride = a.dest_stride;
    p.x_rank_stride = a.x_rank_stride;
    p.amax_rank_stride = a.amax_rank_stride;
    p.send_rank_stride = a.send_rank_stride;
    p.B = a.B;
    p.L = a.L;
    p.H = a.H;
    p.P = a.P;
    p.h = a.H / a.P;
    p.slots = slots_of(a.L);
    p.sec = chunk_section(a.B, a.L, p.h, a.D);
    p.ssec = chunk_scale_section(a.B, a.L, p.h);
    p.rank0 = a.rank0;
    constexpr int HB = 512 / D;
    p.nhb = (int)((a.H + HB - 1) / HB);
    dim3 grid((unsigned)(a.B * p.slots * p.nhb), 1, (unsigned)a.nranks);
    hipLaunchKernelGGL((pack_kernel<DT, D>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64>(a, stream)
                                           : launch_t<kBF16, 128>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64>(a, stream) : launch_t<kFP16, 128>(a, stream);
}

}  // namespace ulp
