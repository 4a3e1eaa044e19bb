// unpack.hip -- received chunks -> SageAttention input layouts (gfx950).
//
// flashinfer.comm._ulysses_lowp.unpack_for_sage (description, Returns): the destination's
// P source chunks become
//   q8, k8  int8 [B, S, h, D]  in logical (global row) order,
//   v8      E4M3 [B, D, h, Spad], Spad = ceil(S/64)*64, columns [S, Spad) zero,
//   q_scale, k_scale fp32 [B, h, W], W = ceil(n/64) for the consumer's live prefix n.
// One launch does all three parts; each workgroup picks its part from its block index:
//   * copy:  every (tensor, source, b) block of L*h*D bytes is contiguous on both sides, so
//            it is a plain 16-byte vector copy (4 vectors per thread per workgroup);
//   * V:     each wave transposes a 16-row x 16-byte register block per lane: 16 coalesced
//            16-byte loads along channels, 16 byte-level 4x4 transposes with v_perm_b32,
//            16 coalesced 16-byte stores along time.  A wave covers 128 (D = 128) or 256
//            (D = 64) time steps x all D channels of one (b, head); rows are fetched from
//            whichever source holds them, so tiles that straddle shards need no special case;
//   * scales: group g's scale is read from the source holding its first row, floor(64g/L).
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

#ifndef ULP_UNPACK_COPY_UNROLL
#define ULP_UNPACK_COPY_UNROLL 4
#endif
constexpr int kCopyUnroll = ULP_UNPACK_COPY_UNROLL;

struct UnpackParams {
    const uint8_t* recv;
    int64_t recv_dest_stride;
    int8_t *q8, *k8;
    uint8_t* v8;
    float *q_scale, *k_scale;
    int64_t qk_dest_stride, v_dest_stride, scale_dest_stride;
    int64_t B, L, h, P, S, spad, W, slots, cb, sec, ssec, seg_vecs;
    int64_t copy_bps, n_copy, n_v, v_tiles;
};

template <int D, bool NT>
__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackParams p) {
    const int64_t z = blockIdx.z;
    const uint8_t* recv = p.recv + z * p.recv_dest_stride;
    const int tid = threadIdx.x;
    int64_t bid = blockIdx.x;
    const int64_t L = p.L, h = p.h;

    if (bid < p.n_copy) {
        const int64_t seg = bid / p.copy_bps, part = bid % p.copy_bps;
        const int64_t tensor = seg / (p.P * p.B);
        const int64_t s = (seg / p.B) % p.P, b = seg % p.B;
        const uint8_t* src = recv + s * p.cb + tensor * p.sec + b * L * h * D;
        int8_t* dst = (tensor ? p.k8 : p.q8) + z * p.qk_dest_stride + (b * p.S + s * L) * h * D;
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int i = 0; i < kCopyUnroll; ++i) {
            const int64_t e = (part * kCopyUnroll + i) * kThreads + tid;
            if (e < p.seg_vecs) v[i] = load16<true>(src + 16 * e);
        }
#pragma unroll
        for (int i = 0; i < kCopyUnroll; ++i) {
            const int64_t e = (part * kCopyUnroll + i) * kThreads + tid;
            if (e < p.seg_vecs) store16<NT>(dst + 16 * e, v[i]);
        }
        return;
    }
    bid -= p.n_copy;

    if (bid < p.n_v) {
        constexpr int DB = D / 16;             // 16-byte channel blocks per row
        constexpr int T = 16 * (64 / DB);      // time steps per wave tile
        const int wave = tid >> 6, lane = tid & 63;
        const int64_t item = bid * 4 + wave;   // (b, head, tile)
        if (item >= p.B * h * p.v_tiles) return;
        const int64_t tile = item % p.v_tiles, bj = item / p.v_tiles;
        const int64_t j = bj % h, b = bj / h;
        const int db = lane % DB, tb = lane / DB;
        const int64_t t0 = tile * T + tb * 16;
        if (t0 >= p.spad) return;
        const int d0 = db * 16;

        uint32_t w[16][4];
        int64_t s = t0 / L, l = t0 % L;
        const uint8_t* vsec = recv + 2 * p.sec + ((b * L) * h + j) * D + d0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (t0 + i < p.S) x = load16<true>(vsec + s * p.cb + l * h * D);
            w[i][0] = x.x;
            w[i][1] = x.y;
            w[i][2] = x.z;
            w[i][3] = x.w;
            if (++l == L) {
                l = 0;
                ++s;
            }
        }
        uint32_t o[16][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                transpose4x4(w[4 * m][k], w[4 * m + 1][k], w[4 * m + 2][k], w[4 * m + 3][k],
                             o[4 * k][m], o[4 * k + 1][m], o[4 * k + 2][m], o[4 * k + 3][m]);
        uint8_t* out = p.v8 + z * p.v_dest_stride + ((b * D + d0) * h + j) * p.spad + t0;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc)
            store16<NT>(out + (int64_t)cc * h * p.spad, make_uint4(o[cc][0], o[cc][1], o[cc][2], o[cc][3]));
        return;
    }
    bid -= p.n_v;

    const int64_t item = bid * kThreads + tid;   // (b, head, g)
    if (item >= p.B * h * p.W) return;
    const int64_t g = item % p.W, bj = item / p.W;
    const int64_t src = kGroup * g / L;
    const int64_t slot = g - first_group(src, L);
    const uint8_t* c = recv + src * p.cb + 3 * p.sec + 4 * (bj * p.slots + slot);
    p.q_scale[z * p.scale_dest_stride + bj * p.W + g] = *reinterpret_cast<const float*>(c);
    p.k_scale[z * p.scale_dest_stride + bj * p.W + g] =
        *reinterpret_cast<const float*>(c + p.ssec);
}

template <int D>
hipError_t launch_t(const UnpackLaunch& a, hipStream_t stream) {
    UnpackParams p;
    p.recv = a.recv;
    p.recv_dest_stride = a.recv_dest_stride;
    p.q8 = a.q8;
    p.k8 = a.k8;
    p.v8 = a.v8;
    p.q_scale = a.q_scale;
    p.k_scale = a.k_scale;
    p.qk_dest_stride = a.qk_dest_stride;
    p.v_dest_stride = a.v_dest_stride;
    p.scale_dest_stride = a.scale_dest_stride;
    p.B = a.B;
    p.L = a.L;
    p.h = a.h;
    p.P = a.P;
    p.S = a.P * a.L;
    p.spad = (p.S + kGroup - 1) / kGroup * kGroup;
    p.W = a.W;
    p.slots = slots_of(a.L);
    p.cb = chunk_bytes_of(a.B, a.L, a.h, D);
    p.sec = chunk_section(a.B, a.L, a.h, D);
    p.ssec = chunk_scale_section(a.B, a.L, a.h);
    p.seg_vecs = a.L * a.h * D / 16;
    p.copy_bps = (p.seg_vecs + kCopyUnroll * kThreads - 1) / (kCopyUnroll * kThreads);
    p.n_copy = 2 * a.P * a.B * p.copy_bps;
    constexpr int T = 16 * (64 / (D / 16));
    p.v_tiles = (p.spad + T - 1) / T;
    p.n_v = (a.B * a.h * p.v_tiles + 3) / 4;
    const int64_t n_scale = (a.B * a.h * a.W + kThreads - 1) / kThreads;
    dim3 grid((unsigned)(p.n_copy + p.n_v + n_scale), 1, (unsigned)a.ndests);
    // the received chunks are read once (non-temporal); outputs stay cached when small, for
    // the consumer that reads them next
    const int64_t written = a.ndests * (2 * a.B * p.S * a.h * D + a.B * D * a.h * p.spad);
    if (written > kResidentBytes)
        hipLaunchKernelGGL((unpack_kernel<D, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((unpack_kernel<D, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t stream) {
    return a.D == 64 ? launch_t<64>(a, stream) : launch_t<128>(a, stream);
}

// total blocks of one unpack launch (for validation of grid limits)
int64_t unpack_blocks(int64_t B, int64_t L, int64_t h, int64_t D, int64_t P, int64_t W) {
    const int64_t seg_vecs = L * h * D / 16;
    const int64_t bps = (seg_vecs + kCopyUnroll * kThreads - 1) / (kCopyUnroll * kThreads);
    const int64_t S = P * L, spad = (S + kGroup - 1) / kGroup * kGroup;
    const int64_t T = 16 * (64 / (D / 16));
    const int64_t tiles = (spad + T - 1) / T;
    return 2 * P * B * bps + (B * h * tiles + 3) / 4 + (B * h * W + kThreads - 1) / kThreads;
}

}  // namespace ulp
