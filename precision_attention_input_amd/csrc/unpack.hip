// unpack.hip -- received chunks -> SageAttention input layouts (gfx950).
//
// flashinfer.comm._ulysses_lowp.unpack_for_sage (description, Returns): the destination's
// P source chunks become
//   q8, k8  int8 [B, S, h, D]  in logical (global row) order,
//   v8      E4M3 [B, D, h, Spad], Spad = ceil(S/64)*64, columns [S, Spad) zero,
//   q_scale, k_scale fp32 [B, h, W], W = ceil(n/64) for the consumer's live prefix n.
// One launch does all three parts; each workgroup picks its part from its block index:
//   * copy:  every (tensor, source, b) block of L*h*D bytes is contiguous on both sides, so
//            it is a plain 16-byte vector copy (2 or 8 vectors per thread per workgroup);
//   * V:     each wave transposes a 16-row x 16-byte register block per lane: 16 coalesced
//            16-byte loads along channels, 16 byte-level 4x4 transposes with v_perm_b32,
//            16 coalesced 16-byte stores along time.  A wave covers 128 time steps x 128
//            bytes of each row (one head at D = 128, two neighbouring heads at D = 64, so
//            loads are whole cache lines); rows are fetched from whichever source holds
//            them, so tiles that straddle shards need no special case;
//   * scales: group g's scale is read from the source holding its first row, floor(64g/L).
#include "ulp_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

// 16-byte vectors per thread of a copy workgroup, for launches whose received bytes stay
// in the cache (small) and for those streamed from HBM (large).
#ifndef ULP_UNPACK_UNROLL_SMALL
#define ULP_UNPACK_UNROLL_SMALL 8
#endif
#ifndef ULP_UNPACK_UNROLL_LARGE
#define ULP_UNPACK_UNROLL_LARGE 2
#endif
constexpr int kUnrollSmall = ULP_UNPACK_UNROLL_SMALL;
constexpr int kUnrollLarge = ULP_UNPACK_UNROLL_LARGE;

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

// NTL: non-temporal loads of the received chunks.  UNROLL: 16-byte vectors per thread of a
// copy workgroup.  Outputs are always stored non-temporally: they are not read again in
// this path, and streaming stores measured faster than write-allocating ones at every size.
template <int D, bool NTL, int UNROLL>
__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackParams p) {
    const int tid = threadIdx.x;
    const int64_t L = p.L, h = p.h;
    const int64_t z = blockIdx.z;
    int64_t bid = blockIdx.x;
    // Block order within a destination: V transposes first (their waves have the longest
    // load -> transpose -> store chains), then copies, then scales.  Destinations follow
    // one another, so transposes and copies of different destinations overlap.
    if (bid < p.n_v) bid += p.n_copy;
    else if (bid < p.n_v + p.n_copy) bid -= p.n_v;
    const uint8_t* recv = p.recv + z * p.recv_dest_stride;

    if (bid < p.n_copy) {
        const int64_t seg = bid / p.copy_bps, part = bid % p.copy_bps;
        const int64_t tensor = seg / (p.P * p.B);
        const int64_t s = (seg / p.B) % p.P, b = seg % p.B;
        const uint8_t* src = recv + s * p.cb + tensor * p.sec + b * L * h * D;
        int8_t* dst = (tensor ? p.k8 : p.q8) + z * p.qk_dest_stride + (b * p.S + s * L) * h * D;
        uint4 v[UNROLL];
#pragma unroll
        for (int i = 0; i < UNROLL; ++i) {
            const int64_t e = (part * UNROLL + i) * kThreads + tid;
            if (e < p.seg_vecs) v[i] = load16<NTL>(src + 16 * e);
        }
#pragma unroll
        for (int i = 0; i < UNROLL; ++i) {
            const int64_t e = (part * UNROLL + i) * kThreads + tid;
            if (e < p.seg_vecs) store16<true>(dst + 16 * e, v[i]);
        }
        return;
    }
    bid -= p.n_copy;

    if (bid < p.n_v) {
        // Every wave covers 128 bytes of each received row, all channels of one head
        // (D = 128) or of two neighbouring heads (D = 64), so every load is whole 128-byte
        // lines, and 128 time steps: lane (db, tb) holds rows t0 + [0, 16) of channel
        // block db.
        constexpr int HPW = 128 / D;           // heads per wave
        constexpr int T = 128;                 // time steps per wave tile
        const int wave = tid >> 6, lane = tid & 63;
        const int64_t hw = (h + HPW - 1) / HPW;
        const int64_t item = bid * 4 + wave;
        if (item >= p.B * hw * p.v_tiles) return;
        // Wave order: (b, tile, head group) when the received chunks sit in the cache (the
        // four waves of a workgroup then read whole received rows); (b, head group, tile)
        // when they stream from HBM (the waves then write consecutive pieces of the same
        // output rows).
        int64_t tile, jw, b;
        if (NTL) {
            tile = item % p.v_tiles;
            const int64_t bj = item / p.v_tiles;
            jw = bj % hw;
            b = bj / hw;
        } else {
            jw = item % hw;
            const int64_t bt = item / hw;
            tile = bt % p.v_tiles;
            b = bt / p.v_tiles;
        }
        const int db = lane & 7, tb = lane >> 3;
        const int64_t j = jw * HPW + db / (D / 16);
        const int64_t t0 = tile * T + tb * 16;
        if (t0 >= p.spad || j >= h) return;
        const int d0 = (db % (D / 16)) * 16;

        // Rows past the sequence (the zero tail) re-read its last row and are zeroed after
        // the loads: no load sits in a branch, so all 16 are in flight together.
        uint32_t w[16][4];
        const int64_t hD = h * D;
        const int64_t tl = min(t0, p.S - 1);
        const int64_t s0 = tl / L, l0 = tl % L;
        const uint8_t* vsec = recv + 2 * p.sec + ((b * L) * h + j) * D + d0;
        const uint8_t* rlast = vsec + (p.P - 1) * p.cb + (L - 1) * hD;   // row S - 1
        if (L >= 16) {
            // 16 rows cross at most one shard boundary: row i lies in shard s0 while
            // i < L - l0, else in shard s0 + 1.
            const uint8_t* rp0 = vsec + s0 * p.cb + l0 * hD;
            const uint8_t* rp1 = vsec + (s0 + 1) * p.cb + (l0 - L) * hD;
            const int64_t n0 = L - l0, nrow = p.S - t0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint8_t* a = (i < n0 ? rp0 : rp1) + i * hD;
                const uint4 x = load16<NTL>(i < nrow ? a : rlast);
                w[i][0] = x.x;
                w[i][1] = x.y;
                w[i][2] = x.z;
                w[i][3] = x.w;
            }
        } else {
            int64_t s = s0, l = l0;
            const uint8_t* rp = vsec + s * p.cb + l * hD;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint4 x = load16<NTL>(rp);
                w[i][0] = x.x;
                w[i][1] = x.y;
                w[i][2] = x.z;
                w[i][3] = x.w;
                if (t0 + i + 1 < p.S) {        // the next row exists: step to it
                    if (++l == L) {
                        l = 0;
                        ++s;
                        rp = vsec + s * p.cb;
                    } else {
                        rp += hD;
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (t0 + i >= p.S) w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
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
            store16<true>(out + (int64_t)cc * h * p.spad,
                          make_uint4(o[cc][0], o[cc][1], o[cc][2], o[cc][3]));
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

// Geometry of one unpack launch (shared by the launcher and the grid-size validation).
struct UnpackGeometry {
    bool nt_loads;
    int unroll;
    int64_t seg_vecs, copy_bps, n_copy, spad, v_tiles, n_v, n_scale;
};

UnpackGeometry unpack_geometry(int64_t B, int64_t L, int64_t h, int64_t D, int64_t P, int64_t W,
                               int64_t ndests) {
    UnpackGeometry g;
    // received bytes of the launch: streamed from HBM (non-temporal) when they exceed the
    // cache budget, else read through the cache that the pack just wrote them into
    g.nt_loads = ndests * P * chunk_bytes_of(B, L, h, D) > kResidentBytes;
    g.unroll = g.nt_loads ? kUnrollLarge : kUnrollSmall;
    g.seg_vecs = L * h * D / 16;
    g.copy_bps = (g.seg_vecs + g.unroll * kThreads - 1) / (g.unroll * kThreads);
    g.n_copy = 2 * P * B * g.copy_bps;
    const int64_t S = P * L;
    g.spad = (S + kGroup - 1) / kGroup * kGroup;
    const int64_t hw = (h + 128 / D - 1) / (128 / D);   // head groups of 128 bytes
    g.v_tiles = (g.spad + 127) / 128;
    g.n_v = (B * hw * g.v_tiles + 3) / 4;
    g.n_scale = (B * h * W + kThreads - 1) / kThreads;
    return g;
}

template <int D, bool NTL, int UNROLL>
void launch_v(const dim3& grid, hipStream_t stream, const UnpackParams& p) {
    hipLaunchKernelGGL((unpack_kernel<D, NTL, UNROLL>), grid, dim3(kThreads), 0, stream, p);
}

template <int D>
hipError_t launch_t(const UnpackLaunch& a, hipStream_t stream) {
    const UnpackGeometry g = unpack_geometry(a.B, a.L, a.h, D, a.P, a.W, a.ndests);
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
    p.spad = g.spad;
    p.W = a.W;
    p.slots = slots_of(a.L);
    p.cb = chunk_bytes_of(a.B, a.L, a.h, D);
    p.sec = chunk_section(a.B, a.L, a.h, D);
    p.ssec = chunk_scale_section(a.B, a.L, a.h);
    p.seg_vecs = g.seg_vecs;
    p.copy_bps = g.copy_bps;
    p.n_copy = g.n_copy;
    p.v_tiles = g.v_tiles;
    p.n_v = g.n_v;
    dim3 grid((unsigned)(g.n_copy + g.n_v + g.n_scale), 1, (unsigned)a.ndests);
    if (g.nt_loads)
        launch_v<D, true, kUnrollLarge>(grid, stream, p);
    else
        launch_v<D, false, kUnrollSmall>(grid, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t stream) {
    return a.D == 64 ? launch_t<64>(a, stream) : launch_t<128>(a, stream);
}

// total blocks of one unpack launch (for validation of grid limits)
int64_t unpack_blocks(int64_t B, int64_t L, int64_t h, int64_t D, int64_t P, int64_t W,
                      int64_t ndests) {
    const UnpackGeometry g = unpack_geometry(B, L, h, D, P, W, ndests);
    return g.n_copy + g.n_v + g.n_scale;
}

}  // namespace ulp
