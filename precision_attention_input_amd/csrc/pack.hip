// pack.hip -- quantize one rank's shard into per-destination chunks (gfx950).
//
// The pack step the k_grouped_amax page (description) refers to: per global 64-row group a
// scale = RN(amax / 127); every element becomes
//   q8 = clamp(rint(RN(fp32(q) / q_scale)), -127, 127)
//   k8 = clamp(rint(RN(RN(fp32(k) - fp32(mean)) / k_scale)), -127, 127)
//   v8 = E4M3FN(fp32(v)) (nearest even, saturating), or E4M3FN(RN(fp32(v) / v_scale)) with
//        the caller's [B, H, D] V scale (unpack_for_sage Returns: it stays with the caller)
// and lands in the chunk of the destination owning its head (unpack_for_sage Parameters:
// local_heads = H / world_size, contiguous per destination).  Chunk sections: q8, k8, v8
// [B, L, h, D] bytes, then q_scale, k_scale [B, h, slots] fp32, each 256-byte aligned.
//
// Work decomposition: the shard is a [B*L, H*D/16] array of 16-element vectors; one thread
// owns one vector of each of Q, K and V.  It issues all of its loads first (amax of both
// tensors, the K mean, 2 x 16 bytes of each of Q, K, V), then quantizes: centered K and bf16
// Q by the division-free exact decision (quantize_exact in ulp_device.h), fp16 Q by the
// reciprocal fast path with the exact decision as a per-wave fallback when a quotient lies
// near a half-integer; V by the E4M3 conversion.  The arithmetic is kept small enough that
// the kernel is bound by memory alone (32-bit column arithmetic, one IEEE division and one
// v_rcp_f32 per tensor).  A 256-thread workgroup covers kRows rows x kCols vectors, so every
// wave reads and writes whole 1 KB row segments; the grid is (B x row blocks x column
// blocks, ranks), column blocks fastest, so the workgroups in flight cover whole rows.
#include "pack_device.h"
#include "ulp_kernels.h"

namespace ulp {
namespace {

constexpr int kCols = 32;                 // 16-element vectors per workgroup row
constexpr int kRows = kThreads / kCols;   // rows per workgroup

struct PackParams {
    const uint16_t *q, *k, *v, *mean;
    const float *q_amax, *k_amax, *v_scale;
    uint8_t* send;
    int64_t dest_stride, x_rank_stride, amax_rank_stride, send_rank_stride;
    int64_t B, L, H, h, P, slots, sec, ssec;
    uint32_t h_magic;        // floor(x / h) = umulhi(x, h_magic) for x, h < 2^16, h > 1
    int rank0, nranks, row_blocks, col_blocks;   // row_blocks: per batch entry
};

template <int DT, int D, bool NT, bool VS>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p) {
    constexpr int VPH = D / 16;      // 16-element vectors per head row
    const int64_t L = p.L, H = p.H, h = p.h;
    const int64_t rz = blockIdx.z;
    const int64_t rank = p.rank0 + rz;
    uint8_t* send = p.send + rz * p.send_rank_stride;
    const int tid = threadIdx.x;

    if (blockIdx.x == 0) {
        // Zero the padding bytes after each section of every destination chunk.
        const int64_t data = p.B * L * h * D;         // bytes of each code section
        const int64_t sdata = 4 * p.B * h * p.slots;  // bytes of each scale section
        for (int64_t i = tid; i < p.P * 5 * 256; i += kThreads) {
            const int64_t dst = i / (5 * 256), sect = (i / 256) % 5, off = i % 256;
            const int64_t start = sect < 3 ? sect * p.sec + data
                                           : 3 * p.sec + (sect - 3) * p.ssec + sdata;
            const int64_t end = sect < 3 ? (sect + 1) * p.sec : 3 * p.sec + (sect - 2) * p.ssec;
            if (start + off < end) send[dst * p.dest_stride + start + off] = 0;
        }
    }

    // Row (b, l) and 16-element column of this thread; rows < 2^31 and columns < 2^20.
    // Consecutive workgroups take the column blocks of the same rows, so the workgroups in
    // flight read whole rows (contiguous memory) rather than one slice of many rows.
    const uint32_t cblk = blockIdx.x % (uint32_t)p.col_blocks;
    const uint32_t rblk = blockIdx.x / (uint32_t)p.col_blocks;
    const uint32_t b = rblk / (uint32_t)p.row_blocks;
    const uint32_t l = (rblk % (uint32_t)p.row_blocks) * kRows + tid / kCols;
    const uint32_t col = cblk * kCols + tid % kCols;
    if (l >= (uint32_t)L || col >= (uint32_t)(H * VPH)) return;
    const uint32_t head = col / VPH, dv = col % VPH;
    const uint32_t dst = h == 1 ? head : __umulhi(head, p.h_magic);
    const uint32_t jl = head - dst * (uint32_t)h;
    const uint64_t row = (uint64_t)b * (uint64_t)L + l;

    // Issue every load first: amax of both tensors, the K mean, and 2 x 16 bytes of Q, K, V.
    const uint64_t arow = (uint64_t)rz * p.amax_rank_stride + ((uint64_t)b * H + head) * p.slots;
    const int64_t g0 = first_group(rank, L);
    const int64_t g = (rank * L + l) / kGroup;
    const uint32_t j = (uint32_t)(g - g0);
    const float qamax = p.q_amax[arow + j];
    const float kamax = p.k_amax[arow + j];
    const uint64_t xo = (uint64_t)rz * p.x_rank_stride + row * (uint64_t)(H * D) + col * 16;
    const uint4 q0 = load16(p.q + xo);
    const uint4 q1 = load16(p.q + xo + 8);
    const uint4 k0 = load16(p.k + xo);
    const uint4 k1 = load16(p.k + xo + 8);
    // V is read once in the whole path: streamed, so that it does not evict the chunks this
    // launch writes (which the unpack reads next) or Q and K (which the statistics pass
    // just read).  Q and K keep the default policy, which measured faster at every size.
    const uint4 v0 = load16<true>(p.v + xo);
    const uint4 v1 = load16<true>(p.v + xo + 8);
    const uint16_t* mp = p.mean + ((uint64_t)b * H + head) * D + dv * 16;
    const uint4 m0 = load16(mp), m1 = load16(mp + 8);
    float4 sv[4];
    if constexpr (VS) {
        const float4* vp = reinterpret_cast<const float4*>(
            p.v_scale + ((uint64_t)b * H + head) * D + dv * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = vp[i];
    }
    // Keep every load above this point: each wave then has all of its reads in flight at
    // once instead of one tensor's at a time.
    __builtin_amdgcn_sched_barrier(0);

    uint8_t* chunk = send + (uint64_t)dst * p.dest_stride;
    uint8_t* out = chunk + row * (uint64_t)(h * D) + jl * D + dv * 16;
    const QuantScale sq = make_scale(qamax);
    const QuantScale sk = make_scale(kamax);

    store16<NT>(out, quantize16<DT, false, DT == kBF16>(q0, q1, m0, m1, sq));
    store16<NT>(out + p.sec, quantize16<DT, true, true>(k0, k1, m0, m1, sk));
    if constexpr (VS)
        store16<NT>(out + 2 * p.sec, e4m3x16_scaled<DT>(v0, v1, sv));
    else
        store16<NT>(out + 2 * p.sec, e4m3x16<DT>(v0, v1));

    if (dv == 0) {
        // The first row of each touched group writes its scales; row 0 also writes the
        // slots this rank never touches (their amax is passed through like any other).
        float* qs = reinterpret_cast<float*>(chunk + 3 * p.sec) + ((uint64_t)b * h + jl) * p.slots;
        float* ks = reinterpret_cast<float*>(chunk + 3 * p.sec + p.ssec) +
                    ((uint64_t)b * h + jl) * p.slots;
        if (l == max((int64_t)kGroup * g, rank * L) - rank * L) {
            qs[j] = sq.s;
            ks[j] = sk.s;
        }
        if (l == 0) {
            const int64_t n = last_group(rank, L) - g0 + 1;
            for (int64_t jj = n; jj < p.slots; ++jj) {
                qs[jj] = p.q_amax[arow + jj] / 127.0f;
                ks[jj] = p.k_amax[arow + jj] / 127.0f;
            }
        }
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
    p.v_scale = a.v_scale;
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
    // ceil(2^32 / h); exact floor(x / h) for x, h < 2^16 (unused when h == 1)
    p.h_magic = p.h > 1 ? (uint32_t)((((uint64_t)1 << 32) + p.h - 1) / p.h) : 0;
    p.rank0 = a.rank0;
    p.nranks = a.nranks;
    p.row_blocks = (int)((a.L + kRows - 1) / kRows);
    p.col_blocks = (int)((a.H * (a.D / 16) + kCols - 1) / kCols);
    dim3 grid((unsigned)(a.B * p.row_blocks * p.col_blocks), 1, (unsigned)a.nranks);
    const int64_t written = a.nranks * 3 * a.B * a.L * a.H * a.D;   // code bytes of this launch
    const bool nt = written > kResidentBytes;
    const dim3 block(kThreads);
    if (a.v_scale) {
        if (nt) hipLaunchKernelGGL((pack_kernel<DT, D, true, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((pack_kernel<DT, D, false, true>), grid, block, 0, stream, p);
    } else {
        if (nt) hipLaunchKernelGGL((pack_kernel<DT, D, true, false>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((pack_kernel<DT, D, false, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackLaunch& a, hipStream_t stream) {
    if (a.dtype == kBF16) return a.D == 64 ? launch_t<kBF16, 64>(a, stream)
                                           : launch_t<kBF16, 128>(a, stream);
    return a.D == 64 ? launch_t<kFP16, 64>(a, stream) : launch_t<kFP16, 128>(a, stream);
}

}  // namespace ulp
