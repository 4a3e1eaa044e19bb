// ulp_kernels.h -- host-side launch descriptors of the libulp kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulp {

// Grouped amax and/or boundary min/max over one or more ranks' shards, for up to two
// tensors (index 0 and 1 of the arrays; a tensor with x == nullptr is skipped).
struct StatsLaunch {
    const uint16_t* x[2];     // shard of rank rank0 [B, L, H, D]
    const uint16_t* mean[2];  // [B, H, D] or nullptr (raw values)
    float* amax[2];           // [B, H, slots] or nullptr (not wanted)
    float* minmax[2];         // [B, H, 2, 2, D] or nullptr (not wanted)
    int64_t x_rank_stride;    // elements between consecutive ranks' shards
    int64_t amax_rank_stride;
    int64_t minmax_rank_stride;
    int64_t B, L, H, D, P, used;  // used = S when None
    int rank0, nranks, dtype;
};

struct DeriveLaunch {
    float* amax[2];             // [B, H, slots] of rank rank0, updated in place
    const float* minmax[2];     // gathered [P, B, H, 2, 2, D]
    const uint16_t* mean[2];    // [B, H, D] or nullptr (+0)
    int64_t amax_rank_stride;
    int64_t B, H, D, L, P;
    int rank0, nranks, dtype;
};

struct PackLaunch {
    const uint16_t *q, *k, *v, *mean;   // shards of rank rank0 [B, L, H, D]; mean [B, H, D]
    const float *q_amax, *k_amax;       // [B, H, slots] of rank rank0
    const float* v_scale;               // [B, H, D] V divisor (shared by all ranks) or nullptr
    uint8_t* send;                      // chunk (rank0 -> p) at send + p * dest_stride
    int64_t dest_stride;
    int64_t x_rank_stride, amax_rank_stride, send_rank_stride;
    int64_t B, L, H, D, P;
    int rank0, nranks, dtype;
};

// Statistics and pack from one read of the shards (phase 0), and the pack of the slots
// whose amax derive may still change (phase 1, after derive).
struct StatsPackLaunch {
    const uint16_t *q, *k, *v, *mean;   // shards of rank rank0 [B, L, H, D]; mean [B, H, D]
    const float* v_scale;               // [B, H, D] V divisor or nullptr (phase 0)
    float *q_amax, *k_amax;             // [B, H, slots]: written by phase 0, read by phase 1
    float *q_minmax, *k_minmax;         // [B, H, 2, 2, D] (phase 0)
    uint8_t* send;                      // chunk (rank0 -> p) at send + p * dest_stride
    int64_t dest_stride;
    int64_t x_rank_stride, amax_rank_stride, minmax_rank_stride, send_rank_stride;
    int64_t B, L, H, D, P, used;        // used = S when None
    int rank0, nranks, dtype, phase;
};

struct UnpackLaunch {
    const uint8_t* recv;           // [P, chunk_bytes] of destination 0 of this launch
    int64_t recv_dest_stride;      // bytes between consecutive destinations' recv blocks
    int8_t *q8, *k8;
    uint8_t* v8;
    float *q_scale, *k_scale;
    int64_t qk_dest_stride, v_dest_stride, scale_dest_stride;   // elements per destination
    int64_t B, L, h, D, P, W;
    int ndests;
};

struct KMeanLaunch {
    const uint16_t* k;        // stacked shards [P, B, L, H, D]
    double* workspace;        // [kmean_chunks(B, H, D, used), B, H*D] binary64
    float* mean_f32;          // [B, H, D]
    uint16_t* mean_dtype;     // [B, H, D] or nullptr
    int64_t B, L, H, D, used;
    int dtype;
};

// K statistics and the K mean from one read of the stacked K shards.
struct KStatsLaunch {
    const uint16_t* k;        // [P, B, L, H, D]
    uint16_t* mm;             // workspace [P, B, H, slots, 2, D] raw 16-bit min / max
    double* sum;              // workspace [P, B, H, slots, D]
    float* minmax;            // [P, B, H, 2, 2, D]
    float* amax;              // [P, B, H, slots]
    float* mean_f32;          // [B, H, D]
    uint16_t* mean_dtype;     // [B, H, D]
    int64_t B, L, H, D, P, used;
    int dtype;
};

// Attention over one destination's unpacked tensors (the consumer check).
struct ConsumerLaunch {
    const int8_t *q8, *k8;         // [B, S, h, D]
    const uint8_t* v8;             // [B, D, h, Spad] E4M3
    const float *q_scale, *k_scale;   // [B, h, W]
    const float* v_scale;          // [B, h, D] or nullptr
    float* out;                    // [B, used, h, D]
    int64_t B, S, h, D, W, used;
};

// Bytes of the device scratch array of the entry points that allocate nothing, and its
// address on the current device (looked up once per device).
constexpr int64_t kScratchBytes = (int64_t)16 << 20;
hipError_t scratch_pointer(void** out);

// Rows per partial sum of the K mean, and the number of such chunks (workspace rows).
int64_t kmean_rows(int64_t B, int64_t H, int64_t D, int64_t used);
int64_t kmean_chunks(int64_t B, int64_t H, int64_t D, int64_t used);

hipError_t launch_stats(const StatsLaunch& a, hipStream_t stream);
hipError_t launch_kmean(const KMeanLaunch& a, hipStream_t stream);
hipError_t launch_consumer(const ConsumerLaunch& a, hipStream_t stream);
hipError_t launch_kstats(const KStatsLaunch& a, hipStream_t stream);
hipError_t launch_derive(const DeriveLaunch& a, hipStream_t stream);
hipError_t launch_pack(const PackLaunch& a, hipStream_t stream);
hipError_t launch_stats_pack(const StatsPackLaunch& a, hipStream_t stream);
hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t stream);

// Geometry shared by host and kernels.
inline int64_t slots_of(int64_t L) { return L % 64 == 0 ? L / 64 : (L + 63) / 64 + 1; }
inline int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }
inline int64_t chunk_section(int64_t B, int64_t L, int64_t h, int64_t D) {
    return align256(B * L * h * D);
}
inline int64_t chunk_scale_section(int64_t B, int64_t L, int64_t h) {
    return align256(4 * B * h * slots_of(L));
}
// workspace of the one-read K statistics: sums (fp64), then the raw 16-bit min / max, per
// (rank, b, head, slot, channel)
inline int64_t kstats_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t D, int64_t P) {
    return P * B * H * slots_of(L) * D * (8 + 2 * 2);
}
inline int64_t chunk_bytes_of(int64_t B, int64_t L, int64_t h, int64_t D) {
    return 3 * chunk_section(B, L, h, D) + 2 * chunk_scale_section(B, L, h);
}

}  // namespace ulp
