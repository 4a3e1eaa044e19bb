// api.hip -- the C ABI of libulp: argument validation and kernel launches.
//
// Every entry point validates all of its arguments on the host before launching anything;
// an invalid call returns an error code, launches nothing and leaves a message for
// ulp_last_error().  No entry point allocates device memory or synchronizes the host.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "ulp.h"
#include "ulp_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ULP_ELAUNCH, "%s: kernel launch failed: %s", what,
                                     hipGetErrorString(e));
    return ULP_OK;
}

constexpr int64_t kMaxGrid = (int64_t)1 << 31;

// Shared domain checks (pages: world_size one of 2/4/6/8, head_dim 64 or 128, H divisible
// by world_size).  rank < 0 skips the rank check.
int check_shape(const char* fn, int dtype, int64_t B, int64_t L, int64_t H, int64_t D, int P,
                int rank, bool check_rank) {
    if (dtype != ULP_BF16 && dtype != ULP_FP16)
        return fail(ULP_EINVAL, "%s: dtype must be ULP_BF16 (0) or ULP_FP16 (1), got %d", fn,
                    dtype);
    if (D != 64 && D != 128)
        return fail(ULP_EUNSUPPORTED, "%s: head_dim must be 64 or 128, got %lld", fn,
                    (long long)D);
    if (P != 2 && P != 4 && P != 6 && P != 8)
        return fail(ULP_EUNSUPPORTED, "%s: world_size must be 2, 4, 6 or 8, got %d", fn, P);
    if (check_rank && (rank < 0 || rank >= P))
        return fail(ULP_EINVAL, "%s: rank %d outside [0, %d)", fn, rank, P);
    if (B < 1 || L < 1 || H < 1)
        return fail(ULP_EINVAL, "%s: batch, local_sequence and heads must be >= 1 "
                                "(got B=%lld L=%lld H=%lld)", fn, (long long)B, (long long)L,
                    (long long)H);
    if (H > 65535)
        return fail(ULP_EINVAL, "%s: at most 65535 heads, got %lld", fn, (long long)H);
    if (H % P != 0)
        return fail(ULP_EINVAL, "%s: heads %lld not divisible by world_size %d", fn,
                    (long long)H, P);
    // Keep every element offset far from int64 overflow and every grid within HIP limits.
    const int64_t lim = (int64_t)1 << 40;
    if (B > lim / L || B * L > lim / H || B * L * H > lim / (D * P))
        return fail(ULP_EINVAL, "%s: problem too large", fn);
    const int64_t slots = ulp::slots_of(L);
    if (B * slots * ((H + 1) / 2) >= kMaxGrid ||
        B * ((L + 7) / 8) * ((H * D + 511) / 512) >= kMaxGrid)
        return fail(ULP_EINVAL, "%s: problem too large for one launch", fn);
    return ULP_OK;
}

int check_seq(const char* fn, const char* name, int64_t v, int64_t S) {
    if (v == ULP_NONE || (v >= 1 && v <= S)) return ULP_OK;
    return fail(ULP_EINVAL, "%s: %s must be ULP_NONE or in [1, %lld], got %lld", fn, name,
                (long long)S, (long long)v);
}

int check_ptr(const char* fn, const char* name, const void* p, int align = 16) {
    if (p == nullptr) return fail(ULP_EINVAL, "%s: %s is NULL", fn, name);
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
        return fail(ULP_EALIGN, "%s: %s is not %d-byte aligned", fn, name, align);
    return ULP_OK;
}

int check_aligned_flag(const char* fn, int aligned, int64_t L) {
    if (aligned != ULP_NONE && aligned != 0 && aligned != 1)
        return fail(ULP_EINVAL, "%s: aligned must be ULP_NONE, 0 or 1, got %d", fn, aligned);
    if (aligned == 1 && L % 128 != 0)
        return fail(ULP_EINVAL, "%s: aligned=True requires local_sequence %% 128 == 0 "
                                "(local_sequence=%lld)", fn, (long long)L);
    return ULP_OK;
}

#define TRY(expr)                  \
    do {                           \
        int rc_ = (expr);          \
        if (rc_ != ULP_OK) return rc_; \
    } while (0)

int64_t used_or_s(int64_t used, int64_t S) { return used == ULP_NONE ? S : used; }
int64_t width_of(int64_t n) { return (n + ULP_GROUP_ROWS - 1) / ULP_GROUP_ROWS; }

}  // namespace

namespace ulp {
int64_t unpack_blocks(int64_t B, int64_t L, int64_t h, int64_t D, int64_t P, int64_t W,
                      int64_t ndests);
}

extern "C" {

int64_t ulp_slots(int64_t local_sequence) {
    return local_sequence < 1 ? 0 : ulp::slots_of(local_sequence);
}

int ulp_scale_widths(int64_t n, int64_t* q_width, int64_t* k_width) {
    if (n < 1) return fail(ULP_EINVAL, "ulp_scale_widths: n must be >= 1, got %lld", (long long)n);
    if (!q_width || !k_width) return fail(ULP_EINVAL, "ulp_scale_widths: NULL output");
    *q_width = width_of(n);
    *k_width = width_of(n);
    return ULP_OK;
}

int64_t ulp_chunk_bytes(int64_t B, int64_t L, int64_t h, int64_t D) {
    if (B < 1 || L < 1 || h < 1 || D < 1) return 0;
    return ulp::chunk_bytes_of(B, L, h, D);
}

const char* ulp_last_error(void) { return g_last_error.c_str(); }

int ulp_k_grouped_amax(const void* x, const void* k_mean, int dtype, int64_t B, int64_t L,
                       int64_t H, int64_t D, int rank, int world_size, int64_t used_sequence,
                       float* out, void* stream) {
    const char* fn = "ulp_k_grouped_amax";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, rank, true));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "x", x));
    if (k_mean) TRY(check_ptr(fn, "k_mean", k_mean));
    TRY(check_ptr(fn, "out", out));
    ulp::StatsLaunch a{};
    a.x[0] = static_cast<const uint16_t*>(x);
    a.mean[0] = static_cast<const uint16_t*>(k_mean);
    a.amax[0] = out;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.used = used_or_s(used_sequence, world_size * L);
    a.rank0 = rank; a.nranks = 1; a.dtype = dtype;
    return launched(ulp::launch_stats(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_boundary_minmax(const void* x, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
                        int rank, int world_size, int64_t used_sequence, float* out,
                        void* stream) {
    const char* fn = "ulp_boundary_minmax";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, rank, true));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "x", x));
    TRY(check_ptr(fn, "out", out));
    ulp::StatsLaunch a{};
    a.x[0] = static_cast<const uint16_t*>(x);
    a.minmax[0] = out;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.used = used_or_s(used_sequence, world_size * L);
    a.rank0 = rank; a.nranks = 1; a.dtype = dtype;
    return launched(ulp::launch_stats(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_derive_k_boundary_amax(float* grouped_amax, const float* gathered_minmax,
                               const void* k_mean, int dtype, int64_t B, int64_t H, int64_t D,
                               int rank, int64_t local_sequence, int world_size, void* stream) {
    const char* fn = "ulp_derive_k_boundary_amax";
    TRY(check_shape(fn, dtype, B, local_sequence, H, D, world_size, rank, true));
    TRY(check_ptr(fn, "grouped_amax", grouped_amax));
    TRY(check_ptr(fn, "gathered_minmax", gathered_minmax));
    if (k_mean) TRY(check_ptr(fn, "k_mean", k_mean));
    ulp::DeriveLaunch a{};
    a.amax[0] = grouped_amax;
    a.minmax[0] = gathered_minmax;
    a.mean[0] = static_cast<const uint16_t*>(k_mean);
    a.B = B; a.H = H; a.D = D; a.L = local_sequence; a.P = world_size;
    a.rank0 = rank; a.nranks = 1; a.dtype = dtype;
    return launched(ulp::launch_derive(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
             const float* q_amax, const float* k_amax, const float* v_scale, int64_t B,
             int64_t L, int64_t H, int64_t D, int rank, int world_size, uint8_t* send,
             int64_t dest_stride_bytes, void* stream) {
    const char* fn = "ulp_pack";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, rank, true));
    TRY(check_ptr(fn, "q", q));
    TRY(check_ptr(fn, "k", k));
    TRY(check_ptr(fn, "v", v));
    TRY(check_ptr(fn, "k_mean", k_mean));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    if (v_scale) TRY(check_ptr(fn, "v_scale", v_scale));
    TRY(check_ptr(fn, "send", send));
    const int64_t cb = ulp::chunk_bytes_of(B, L, H / world_size, D);
    if (dest_stride_bytes % 256 != 0)
        return fail(ULP_EALIGN, "%s: dest_stride_bytes %lld is not a multiple of 256", fn,
                    (long long)dest_stride_bytes);
    if (dest_stride_bytes < cb)
        return fail(ULP_EINVAL, "%s: dest_stride_bytes %lld is smaller than the chunk (%lld)",
                    fn, (long long)dest_stride_bytes, (long long)cb);
    ulp::PackLaunch a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.mean = static_cast<const uint16_t*>(k_mean);
    a.q_amax = q_amax;
    a.k_amax = k_amax;
    a.v_scale = v_scale;
    a.send = send;
    a.dest_stride = dest_stride_bytes;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.rank0 = rank; a.nranks = 1; a.dtype = dtype;
    return launched(ulp::launch_pack(a, static_cast<hipStream_t>(stream)), fn);
}

static int unpack_common(const char* fn, const uint8_t* recv, int64_t B, int64_t L, int64_t h,
                         int64_t D, int world_size, int aligned, int64_t scale_sequence,
                         int8_t* q8, int8_t* k8, uint8_t* v8, float* q_scale, float* k_scale,
                         int ndests, void* stream) {
    if (h < 1) return fail(ULP_EINVAL, "%s: local_heads must be >= 1, got %lld", fn, (long long)h);
    TRY(check_shape(fn, ULP_BF16, B, L, h * world_size, D, world_size, 0, false));
    TRY(check_aligned_flag(fn, aligned, L));
    const int64_t S = world_size * L;
    TRY(check_seq(fn, "scale_sequence", scale_sequence, S));
    TRY(check_ptr(fn, "recv", recv));
    TRY(check_ptr(fn, "q8", q8));
    TRY(check_ptr(fn, "k8", k8));
    TRY(check_ptr(fn, "v8", v8));
    TRY(check_ptr(fn, "q_scale", q_scale));
    TRY(check_ptr(fn, "k_scale", k_scale));
    const int64_t W = width_of(scale_sequence == ULP_NONE ? S : scale_sequence);
    if (ulp::unpack_blocks(B, L, h, D, world_size, W, ndests) >= kMaxGrid)
        return fail(ULP_EINVAL, "%s: problem too large for one launch", fn);
    const int64_t spad = (S + ULP_GROUP_ROWS - 1) / ULP_GROUP_ROWS * ULP_GROUP_ROWS;
    const int64_t cb = ulp::chunk_bytes_of(B, L, h, D);
    ulp::UnpackLaunch a{};
    a.recv = recv;
    a.recv_dest_stride = (int64_t)world_size * cb;
    a.q8 = q8;
    a.k8 = k8;
    a.v8 = v8;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.qk_dest_stride = B * S * h * D;
    a.v_dest_stride = B * D * h * spad;
    a.scale_dest_stride = B * h * W;
    a.B = B; a.L = L; a.h = h; a.D = D; a.P = world_size; a.W = W;
    a.ndests = ndests;
    return launched(ulp::launch_unpack(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_unpack_for_sage(const uint8_t* recv, int64_t B, int64_t L, int64_t h, int64_t D,
                        int world_size, int aligned, int64_t scale_sequence, int8_t* q8,
                        int8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, void* stream) {
    return unpack_common("ulp_unpack_for_sage", recv, B, L, h, D, world_size, aligned,
                         scale_sequence, q8, k8, v8, q_scale, k_scale, 1, stream);
}

int ulp_group_stats(const void* q, const void* k, const void* k_mean, int dtype, int64_t B,
                    int64_t L, int64_t H, int64_t D, int world_size, int64_t used_sequence,
                    float* q_amax, float* k_amax, float* q_minmax, float* k_minmax,
                    void* stream) {
    const char* fn = "ulp_group_stats";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, 0, false));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "q", q));
    TRY(check_ptr(fn, "k", k));
    TRY(check_ptr(fn, "k_mean", k_mean));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    TRY(check_ptr(fn, "q_minmax", q_minmax));
    TRY(check_ptr(fn, "k_minmax", k_minmax));
    ulp::StatsLaunch a{};
    a.x[0] = static_cast<const uint16_t*>(q);
    a.x[1] = static_cast<const uint16_t*>(k);
    a.mean[1] = static_cast<const uint16_t*>(k_mean);
    a.amax[0] = q_amax;
    a.amax[1] = k_amax;
    a.minmax[0] = q_minmax;
    a.minmax[1] = k_minmax;
    a.x_rank_stride = B * L * H * D;
    a.amax_rank_stride = B * H * ulp::slots_of(L);
    a.minmax_rank_stride = B * H * 4 * D;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.used = used_or_s(used_sequence, world_size * L);
    a.rank0 = 0; a.nranks = world_size; a.dtype = dtype;
    return launched(ulp::launch_stats(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_group_derive(float* q_amax, float* k_amax, const float* q_minmax,
                     const float* k_minmax, const void* k_mean, int dtype, int64_t B,
                     int64_t H, int64_t D, int64_t local_sequence, int world_size,
                     void* stream) {
    const char* fn = "ulp_group_derive";
    TRY(check_shape(fn, dtype, B, local_sequence, H, D, world_size, 0, false));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    TRY(check_ptr(fn, "q_minmax", q_minmax));
    TRY(check_ptr(fn, "k_minmax", k_minmax));
    TRY(check_ptr(fn, "k_mean", k_mean));
    ulp::DeriveLaunch a{};
    a.amax[0] = q_amax;
    a.amax[1] = k_amax;
    a.minmax[0] = q_minmax;
    a.minmax[1] = k_minmax;
    a.mean[1] = static_cast<const uint16_t*>(k_mean);
    a.amax_rank_stride = B * H * ulp::slots_of(local_sequence);
    a.B = B; a.H = H; a.D = D; a.L = local_sequence; a.P = world_size;
    a.rank0 = 0; a.nranks = world_size; a.dtype = dtype;
    return launched(ulp::launch_derive(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_group_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
                   const float* q_amax, const float* k_amax, const float* v_scale, int64_t B,
                   int64_t L, int64_t H, int64_t D, int world_size, uint8_t* group,
                   void* stream) {
    const char* fn = "ulp_group_pack";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, 0, false));
    TRY(check_ptr(fn, "q", q));
    TRY(check_ptr(fn, "k", k));
    TRY(check_ptr(fn, "v", v));
    TRY(check_ptr(fn, "k_mean", k_mean));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    if (v_scale) TRY(check_ptr(fn, "v_scale", v_scale));
    TRY(check_ptr(fn, "group", group));
    const int64_t cb = ulp::chunk_bytes_of(B, L, H / world_size, D);
    ulp::PackLaunch a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.mean = static_cast<const uint16_t*>(k_mean);
    a.q_amax = q_amax;
    a.k_amax = k_amax;
    a.v_scale = v_scale;
    a.send = group;
    a.dest_stride = (int64_t)world_size * cb;
    a.x_rank_stride = B * L * H * D;
    a.amax_rank_stride = B * H * ulp::slots_of(L);
    a.send_rank_stride = cb;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.rank0 = 0; a.nranks = world_size; a.dtype = dtype;
    return launched(ulp::launch_pack(a, static_cast<hipStream_t>(stream)), fn);
}

// Shared part of the one-read statistics + pack entry points (phase 0) and of the pack of
// the slots that wait for derive (phase 1).
static int stats_pack_common(const char* fn, int phase, const void* q, const void* k,
                             const void* v, const void* k_mean, int dtype,
                             const float* v_scale, int64_t B, int64_t L, int64_t H, int64_t D,
                             int rank, int nranks, int world_size, int64_t used_sequence,
                             float* q_amax, float* k_amax, float* q_minmax, float* k_minmax,
                             uint8_t* send, int64_t dest_stride_bytes,
                             int64_t send_rank_stride, void* stream) {
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, rank, nranks == 1));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "q", q));
    TRY(check_ptr(fn, "k", k));
    if (phase == 0) TRY(check_ptr(fn, "v", v));
    TRY(check_ptr(fn, "k_mean", k_mean));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    TRY(check_ptr(fn, "q_minmax", q_minmax));
    TRY(check_ptr(fn, "k_minmax", k_minmax));
    if (phase == 0 && v_scale) TRY(check_ptr(fn, "v_scale", v_scale));
    TRY(check_ptr(fn, "send", send));
    const int64_t cb = ulp::chunk_bytes_of(B, L, H / world_size, D);
    if (dest_stride_bytes % 256 != 0)
        return fail(ULP_EALIGN, "%s: dest_stride_bytes %lld is not a multiple of 256", fn,
                    (long long)dest_stride_bytes);
    if (dest_stride_bytes < cb)
        return fail(ULP_EINVAL, "%s: dest_stride_bytes %lld is smaller than the chunk (%lld)",
                    fn, (long long)dest_stride_bytes, (long long)cb);
    if (B * ulp::slots_of(L) * (H * D / 128) + B * ((L + 7) / 8) * ((H * D + 511) / 512) >=
        kMaxGrid)
        return fail(ULP_EINVAL, "%s: problem too large for one launch", fn);
    ulp::StatsPackLaunch a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.mean = static_cast<const uint16_t*>(k_mean);
    a.v_scale = v_scale;
    a.q_amax = q_amax;
    a.k_amax = k_amax;
    a.q_minmax = q_minmax;
    a.k_minmax = k_minmax;
    a.send = send;
    a.dest_stride = dest_stride_bytes;
    a.x_rank_stride = B * L * H * D;
    a.amax_rank_stride = B * H * ulp::slots_of(L);
    a.minmax_rank_stride = B * H * 4 * D;
    a.send_rank_stride = send_rank_stride;
    a.B = B; a.L = L; a.H = H; a.D = D; a.P = world_size;
    a.used = used_or_s(used_sequence, world_size * L);
    a.rank0 = nranks == 1 ? rank : 0;
    a.nranks = nranks;
    a.dtype = dtype;
    a.phase = phase;
    return launched(ulp::launch_stats_pack(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_stats_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
                   const float* v_scale, int64_t B, int64_t L, int64_t H, int64_t D, int rank,
                   int world_size, int64_t used_sequence, float* q_amax, float* k_amax,
                   float* q_minmax, float* k_minmax, uint8_t* send, int64_t dest_stride_bytes,
                   void* stream) {
    return stats_pack_common("ulp_stats_pack", 0, q, k, v, k_mean, dtype, v_scale, B, L, H, D,
                             rank, 1, world_size, used_sequence, q_amax, k_amax, q_minmax,
                             k_minmax, send, dest_stride_bytes, 0, stream);
}

int ulp_derive_pack(const void* q, const void* k, const void* k_mean, int dtype, float* q_amax,
                    float* k_amax, const float* q_minmax, const float* k_minmax, int64_t B,
                    int64_t L, int64_t H, int64_t D, int rank, int world_size,
                    int64_t used_sequence, uint8_t* send, int64_t dest_stride_bytes,
                    void* stream) {
    return stats_pack_common("ulp_derive_pack", 1, q, k, nullptr, k_mean, dtype, nullptr, B, L,
                             H, D, rank, 1, world_size, used_sequence, q_amax, k_amax,
                             const_cast<float*>(q_minmax), const_cast<float*>(k_minmax), send,
                             dest_stride_bytes, 0, stream);
}

int ulp_group_stats_pack(const void* q, const void* k, const void* v, const void* k_mean,
                         int dtype, const float* v_scale, int64_t B, int64_t L, int64_t H,
                         int64_t D, int world_size, int64_t used_sequence, float* q_amax,
                         float* k_amax, float* q_minmax, float* k_minmax, uint8_t* group,
                         void* stream) {
    const int64_t cb = ulp::chunk_bytes_of(B, L, H / (world_size > 0 ? world_size : 1), D);
    return stats_pack_common("ulp_group_stats_pack", 0, q, k, v, k_mean, dtype, v_scale, B, L,
                             H, D, 0, world_size, world_size, used_sequence, q_amax, k_amax,
                             q_minmax, k_minmax, group, (int64_t)world_size * cb, cb, stream);
}

int ulp_group_derive_pack(const void* q, const void* k, const void* k_mean, int dtype,
                          float* q_amax, float* k_amax, const float* q_minmax,
                          const float* k_minmax, int64_t B, int64_t L, int64_t H, int64_t D,
                          int world_size, int64_t used_sequence, uint8_t* group, void* stream) {
    const int64_t cb = ulp::chunk_bytes_of(B, L, H / (world_size > 0 ? world_size : 1), D);
    return stats_pack_common("ulp_group_derive_pack", 1, q, k, nullptr, k_mean, dtype, nullptr,
                             B, L, H, D, 0, world_size, world_size, used_sequence, q_amax,
                             k_amax, const_cast<float*>(q_minmax), const_cast<float*>(k_minmax),
                             group, (int64_t)world_size * cb, cb, stream);
}

int ulp_group_unpack(const uint8_t* group, int64_t B, int64_t L, int64_t h, int64_t D,
                     int world_size, int aligned, int64_t scale_sequence, int8_t* q8,
                     int8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, void* stream) {
    return unpack_common("ulp_group_unpack", group, B, L, h, D, world_size, aligned,
                         scale_sequence, q8, k8, v8, q_scale, k_scale, world_size, stream);
}

int64_t ulp_k_mean_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t D, int world_size,
                                   int64_t used_sequence) {
    if (B < 1 || L < 1 || H < 1 || D < 1 || world_size < 1) return 0;
    const int64_t S = (int64_t)world_size * L;
    if (used_sequence != ULP_NONE && (used_sequence < 1 || used_sequence > S)) return 0;
    return 8 * B * H * D * ulp::kmean_chunks(B, H, D, used_or_s(used_sequence, S));
}

int ulp_k_mean(const void* k, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
               int world_size, int64_t used_sequence, void* workspace, int64_t workspace_bytes,
               float* mean_f32, void* mean_dtype, void* stream) {
    const char* fn = "ulp_k_mean";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, 0, false));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "k", k));
    TRY(check_ptr(fn, "workspace", workspace));
    TRY(check_ptr(fn, "mean_f32", mean_f32));
    if (mean_dtype) TRY(check_ptr(fn, "mean_dtype", mean_dtype));
    if (B > 65535 || B * H * D / 64 >= kMaxGrid ||
        ulp::kmean_chunks(B, H, D, used_or_s(used_sequence, world_size * L)) > 65535)
        return fail(ULP_EINVAL, "%s: problem too large for one launch", fn);
    const int64_t need = ulp_k_mean_workspace_bytes(B, L, H, D, world_size, used_sequence);
    if (workspace_bytes < need)
        return fail(ULP_EINVAL, "%s: workspace of %lld bytes, %lld needed", fn,
                    (long long)workspace_bytes, (long long)need);
    ulp::KMeanLaunch a{};
    a.k = static_cast<const uint16_t*>(k);
    a.workspace = static_cast<double*>(workspace);
    a.mean_f32 = mean_f32;
    a.mean_dtype = static_cast<uint16_t*>(mean_dtype);
    a.B = B; a.L = L; a.H = H; a.D = D;
    a.used = used_or_s(used_sequence, world_size * L);
    a.dtype = dtype;
    return launched(ulp::launch_kmean(a, static_cast<hipStream_t>(stream)), fn);
}

int ulp_k_mean_noalloc(const void* k, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
                       int world_size, int64_t used_sequence, float* mean_f32,
                       void* mean_dtype, void* stream) {
    const char* fn = "ulp_k_mean_noalloc";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, 0, false));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    const int64_t need = ulp_k_mean_workspace_bytes(B, L, H, D, world_size, used_sequence);
    if (need > ulp::kScratchBytes)
        return fail(ULP_EINVAL, "%s: this shape needs %lld bytes of scratch, more than the "
                                "library's %lld (use ulp_k_mean with a workspace)", fn,
                    (long long)need, (long long)ulp::kScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = ulp::scratch_pointer(&scratch);
    if (e != hipSuccess)
        return fail(ULP_ELAUNCH, "%s: device scratch address: %s", fn, hipGetErrorString(e));
    return ulp_k_mean(k, dtype, B, L, H, D, world_size, used_sequence, scratch,
                      ulp::kScratchBytes, mean_f32, mean_dtype, stream);
}

int64_t ulp_group_stats_with_mean_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t D,
                                                  int world_size) {
    if (B < 1 || L < 1 || H < 1 || D < 1 || world_size < 1) return 0;
    return ulp::kstats_workspace_bytes(B, L, H, D, world_size);
}

int ulp_group_stats_with_mean(const void* q, const void* k, int dtype, int64_t B, int64_t L,
                              int64_t H, int64_t D, int world_size, int64_t used_sequence,
                              void* workspace, int64_t workspace_bytes, float* q_amax,
                              float* k_amax, float* q_minmax, float* k_minmax,
                              float* k_mean_f32, void* k_mean_dtype, void* stream) {
    const char* fn = "ulp_group_stats_with_mean";
    TRY(check_shape(fn, dtype, B, L, H, D, world_size, 0, false));
    TRY(check_seq(fn, "used_sequence", used_sequence, world_size * L));
    TRY(check_ptr(fn, "q", q));
    TRY(check_ptr(fn, "k", k));
    TRY(check_ptr(fn, "workspace", workspace));
    TRY(check_ptr(fn, "q_amax", q_amax));
    TRY(check_ptr(fn, "k_amax", k_amax));
    TRY(check_ptr(fn, "q_minmax", q_minmax));
    TRY(check_ptr(fn, "k_minmax", k_minmax));
    TRY(check_ptr(fn, "k_mean_f32", k_mean_f32));
    TRY(check_ptr(fn, "k_mean_dtype", k_mean_dtype));
    const int64_t need = ulp::kstats_workspace_bytes(B, L, H, D, world_size);
    if (workspace_bytes < need)
        return fail(ULP_EINVAL, "%s: workspace of %lld bytes, %lld needed", fn,
                    (long long)workspace_bytes, (long long)need);
    if ((B * H * D + 15) / 16 >= kMaxGrid || (int64_t)world_size * B * H * ulp::slots_of(L) / 4 >= kMaxGrid)
        return fail(ULP_EINVAL, "%s: problem too large for one launch", fn);
    const int64_t S = world_size * L;
    // Q: grouped amax of raw values and boundary min/max, as ulp_group_stats does
    ulp::StatsLaunch qa{};
    qa.x[0] = static_cast<const uint16_t*>(q);
    qa.amax[0] = q_amax;
    qa.minmax[0] = q_minmax;
    qa.x_rank_stride = B * L * H * D;
    qa.amax_rank_stride = B * H * ulp::slots_of(L);
    qa.minmax_rank_stride = B * H * 4 * D;
    qa.B = B; qa.L = L; qa.H = H; qa.D = D; qa.P = world_size;
    qa.used = used_or_s(used_sequence, S);
    qa.rank0 = 0; qa.nranks = world_size; qa.dtype = dtype;
    const int rc = launched(ulp::launch_stats(qa, static_cast<hipStream_t>(stream)), fn);
    if (rc != ULP_OK) return rc;
    // K: one pass for the per-group min/max, the boundary min/max and the sums; then the
    // mean and the grouped amax
    ulp::KStatsLaunch ka{};
    ka.k = static_cast<const uint16_t*>(k);
    char* ws = static_cast<char*>(workspace);
    ka.sum = reinterpret_cast<double*>(ws);
    ka.mm = reinterpret_cast<uint16_t*>(ws + world_size * B * H * ulp::slots_of(L) * D * 8);
    ka.minmax = k_minmax;
    ka.amax = k_amax;
    ka.mean_f32 = k_mean_f32;
    ka.mean_dtype = static_cast<uint16_t*>(k_mean_dtype);
    ka.B = B; ka.L = L; ka.H = H; ka.D = D; ka.P = world_size;
    ka.used = used_or_s(used_sequence, S);
    ka.dtype = dtype;
    return launched(ulp::launch_kstats(ka, static_cast<hipStream_t>(stream)), fn);
}

int ulp_consumer_attention(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           int64_t B, int64_t S, int64_t h, int64_t D, int64_t W,
                           int64_t used, float* out, void* stream) {
    const char* fn = "ulp_consumer_attention";
    if (D != 64 && D != 128)
        return fail(ULP_EUNSUPPORTED, "%s: head_dim must be 64 or 128, got %lld", fn,
                    (long long)D);
    if (B < 1 || S < 1 || h < 1)
        return fail(ULP_EINVAL, "%s: batch, sequence and heads must be >= 1", fn);
    if (used < 1 || used > S)
        return fail(ULP_EINVAL, "%s: used must be in [1, %lld], got %lld", fn, (long long)S,
                    (long long)used);
    if (W < width_of(used))
        return fail(ULP_EINVAL, "%s: scale width %lld < ceil(used / 64) = %lld", fn,
                    (long long)W, (long long)width_of(used));
    if (B > 65535 || h > 65535 || B * S > ((int64_t)1 << 40) / (h * D))
        return fail(ULP_EINVAL, "%s: problem too large", fn);
    const int64_t spad = width_of(S) * ULP_GROUP_ROWS;
    if (S * h * D >= ((int64_t)1 << 31) || D * h * spad >= ((int64_t)1 << 31))
        return fail(ULP_EINVAL, "%s: one batch entry of k8 or v8 is 2 GiB or more", fn);
    TRY(check_ptr(fn, "q8", q8));
    TRY(check_ptr(fn, "k8", k8));
    TRY(check_ptr(fn, "v8", v8));
    TRY(check_ptr(fn, "q_scale", q_scale, 4));   // read one float at a time
    TRY(check_ptr(fn, "k_scale", k_scale, 4));
    if (v_scale) TRY(check_ptr(fn, "v_scale", v_scale));
    TRY(check_ptr(fn, "out", out));
    ulp::ConsumerLaunch a{};
    a.q8 = q8;
    a.k8 = k8;
    a.v8 = v8;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.out = out;
    a.B = B; a.S = S; a.h = h; a.D = D; a.W = W; a.used = used;
    return launched(ulp::launch_consumer(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
