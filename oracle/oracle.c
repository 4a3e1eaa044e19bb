/*
 * oracle.c -- plain CPU oracle of the smooth-K low-precision Ulysses pack/unpack.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (libulp.so and
 * its Python binding) never links, imports or calls it, and shares no code with it.
 *
 * It follows the per-rank pipeline exactly as the FlashInfer pages describe it, one
 * step per function, with plain loops, single-threaded, in IEEE fp32:
 *
 *   ora_k_grouped_amax          flashinfer.comm._ulysses_lowp.k_grouped_amax (description,
 *                               Returns): partial amax of |K - mean| per touched global
 *                               64-row group, with the partial-live-group fix.
 *   ora_boundary_minmax         flashinfer.comm._ulysses_lowp.derive_k_boundary_amax
 *                               (description, gathered_minmax parameter): the raw min/max
 *                               payload of the stats all-gather.
 *   ora_derive_k_boundary_amax  derive_k_boundary_amax (description, contrib formula).
 *   ora_pack                    per-group scales, INT8 Q / centered K, FP8 E4M3 V, and the
 *                               source-major chunk bytes (k_grouped_amax description names
 *                               the pack kernel's per-group scales; unpack_for_sage
 *                               Parameters name the [world_size, chunk_bytes] buffer).
 *   ora_unpack_for_sage         flashinfer.comm._ulysses_lowp.unpack_for_sage (description,
 *                               Returns).
 *   ora_k_mean                  the global K mean the pages take as an input already rounded
 *                               to the dtype (k_grouped_amax Parameters, k_mean_global): a
 *                               binary64 mean over the live rows, then binary32, then dtype.
 *
 * Floating point: build with -O2 -ffp-contract=off and without -ffast-math on x86-64
 * (SSE arithmetic, FLT_EVAL_METHOD 0): every float operation below is a single IEEE
 * binary32 operation rounded to nearest-even, division is correctly rounded, rintf rounds
 * half to even, subnormals are kept.
 *
 * Readings of points the pages leave open (each is listed with its reason in the design
 * notes of the repository):
 *   - slots(L,64) = L/64 when 64 divides L, else ceil(L/64)+1.  Slot j of rank r is the
 *     global group floor(r*L/64)+j.  Slots a rank does not touch hold the floor 1e-7.
 *   - The boundary min/max runs over live rows (< used) only, after mapping -0 to +0;
 *     an empty slice gives min=+inf, max=-inf.  Layout [B,H,2,2,D]: dim 2 picks the
 *     rank's first (0) or last (1) touched group, dim 3 picks min (0) or max (1).
 *   - Q uses the same machinery with the mean taken as +0 (raw values).
 *   - scale = amax/127; q = clamp(rint(x/scale), -127, 127) with x/scale the IEEE quotient.
 *   - V is converted to OCP E4M3FN, round-to-nearest-even, saturating at 448; unscaled by
 *     default, or divided first (one IEEE binary32 division) by the caller's V scale
 *     [B,H,D] when one is given (unpack_for_sage Returns: the V scale stays with the caller).
 *   - Chunk (source r -> destination p): sections q8, k8, v8 each [B,L,h,D] bytes for
 *     heads p*h..p*h+h-1, then q_scale and k_scale each [B,h,slots] fp32; every section
 *     starts on a 256-byte boundary and padding bytes are 0.
 *   - The scale of global group g is read from the source holding its first row,
 *     floor(64*g/L); widths are ceil(n/64) for both Q and K.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORA_GROUP 64
#define ORA_BF16 0
#define ORA_FP16 1

/* The amax floor: the binary32 value nearest to 1e-7 (k_grouped_amax description). */
static const float ORA_FLOOR = 1e-7f;

/* ------------------------------------------------------------------ decoding inputs */

/* bfloat16 is the upper half of a binary32 pattern. */
static float bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float fp16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    float mag;
    if (e == 0) {
        mag = ldexpf((float)m, -24);                 /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        mag = m ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static float elem(const uint16_t* p, int64_t i, int dtype) {
    return dtype == ORA_BF16 ? bf16_value(p[i]) : fp16_value(p[i]);
}

/* ------------------------------------------------------------------ geometry */

int64_t ora_slots(int64_t L) {
    return (L % ORA_GROUP == 0) ? L / ORA_GROUP : (L + ORA_GROUP - 1) / ORA_GROUP + 1;
}

static int64_t first_group(int64_t rank, int64_t L) { return rank * L / ORA_GROUP; }
static int64_t last_group(int64_t rank, int64_t L) { return (rank * L + L - 1) / ORA_GROUP; }
static int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

int64_t ora_chunk_bytes(int64_t B, int64_t L, int64_t h, int64_t D) {
    return 3 * align256(B * L * h * D) + 2 * align256(4 * B * h * ora_slots(L));
}

/* ------------------------------------------------------------------ encoders */

/* OCP 8-bit floating point, E4M3FN: bias 7, 3 fraction bits, no infinities, largest
 * finite value 448 (code 0x7E), NaN = S.1111.111, subnormal step 2^-9.  Round to nearest
 * even; magnitudes at or above 448 saturate to 448; the sign of zero is kept. */
uint8_t ora_e4m3(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (isnan(x)) return sign | 0x7F;
    if (a >= 448.0f) return sign | 0x7E;
    if (a < 0x1p-6f) {
        /* subnormal range (and zero): integer multiples of 2^-9; n == 8 is 2^-6, code 0x08 */
        float n = rintf(ldexpf(a, 9));
        return sign | (uint8_t)n;
    }
    int e2;
    frexpf(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                 /* a in [2^E, 2^(E+1)), E in [-6, 8] */
    float n = rintf(ldexpf(a, 3 - E));   /* a / 2^(E-3), in [8, 16] */
    if (n == 16.0f) {               /* rounded up into the next binade */
        E += 1;
        n = 8.0f;
    }
    return sign | (uint8_t)(((E + 7) << 3) | ((int)n - 8));
}

/* INT8 with a per-group fp32 scale: clamp(rint(x / scale), -127, 127). */
int8_t ora_quant_i8(float x, float scale) {
    float q = rintf(x / scale);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    return (int8_t)q;
}

/* ------------------------------------------------------------------ step 1: grouped amax */

/* k_grouped_amax (description, Returns).  x: rank's shard [B,L,H,D]; mean: [B,H,D] in the
 * input dtype, or NULL for raw values (Q).  used <= 0 means None.  out: [B,H,slots(L)]. */
void ora_k_grouped_amax(const uint16_t* x, const uint16_t* mean, int dtype, int64_t B,
                        int64_t L, int64_t H, int64_t D, int64_t rank, int64_t P,
                        int64_t used, float* out) {
    int64_t S = P * L;
    int64_t u = used > 0 ? used : S;
    int64_t slots = ora_slots(L);
    int64_t g0 = first_group(rank, L);
    int64_t n = last_group(rank, L) - g0 + 1;
    int64_t partial_live = (u - 1) / ORA_GROUP;
    for (int64_t b = 0; b < B; b++)
        for (int64_t hh = 0; hh < H; hh++)
            for (int64_t j = 0; j < slots; j++) {
                float amax = -INFINITY;
                if (j < n) {
                    int64_t g = g0 + j;
                    int64_t lo = ORA_GROUP * g > rank * L ? ORA_GROUP * g : rank * L;
                    int64_t hi = ORA_GROUP * g + ORA_GROUP < rank * L + L
                                     ? ORA_GROUP * g + ORA_GROUP : rank * L + L;
                    /* the one group that mixes live rows and zero padding: live rows only */
                    if (u < S && g == partial_live && hi > u) hi = u;
                    for (int64_t s = lo; s < hi; s++)
                        for (int64_t d = 0; d < D; d++) {
                            float v = elem(x, ((b * L + (s - rank * L)) * H + hh) * D + d, dtype);
                            float m = mean ? elem(mean, (b * H + hh) * D + d, dtype) : 0.0f;
                            float c = fabsf(v - m);
                            amax = fmaxf(amax, c);
                        }
                }
                out[(b * H + hh) * slots + j] = fmaxf(ORA_FLOOR, amax);
            }
}

/* ------------------------------------------------------------------ step 2: boundary min/max */

/* Raw per-channel min/max over the rank's live rows of its first and last touched group.
 * out: [B,H,2,2,D] fp32 (boundary e, then min/max). */
void ora_boundary_minmax(const uint16_t* x, int dtype, int64_t B, int64_t L, int64_t H,
                         int64_t D, int64_t rank, int64_t P, int64_t used, float* out) {
    int64_t S = P * L;
    int64_t u = used > 0 ? used : S;
    for (int e = 0; e < 2; e++) {
        int64_t g = e == 0 ? first_group(rank, L) : last_group(rank, L);
        int64_t lo = ORA_GROUP * g > rank * L ? ORA_GROUP * g : rank * L;
        int64_t hi = ORA_GROUP * g + ORA_GROUP < rank * L + L ? ORA_GROUP * g + ORA_GROUP
                                                              : rank * L + L;
        if (hi > u) hi = u;
        for (int64_t b = 0; b < B; b++)
            for (int64_t hh = 0; hh < H; hh++)
                for (int64_t d = 0; d < D; d++) {
                    float mn = INFINITY, mx = -INFINITY;
                    for (int64_t s = lo; s < hi; s++) {
                        float v = elem(x, ((b * L + (s - rank * L)) * H + hh) * D + d, dtype);
                        if (v == 0.0f) v = 0.0f;     /* -0 -> +0 */
                        mn = fminf(mn, v);
                        mx = fmaxf(mx, v);
                    }
                    out[(((b * H + hh) * 2 + e) * 2 + 0) * D + d] = mn;
                    out[(((b * H + hh) * 2 + e) * 2 + 1) * D + d] = mx;
                }
    }
}

/* ------------------------------------------------------------------ step 3: derive */

/* derive_k_boundary_amax (description): for each of this rank's first and last touched
 * groups g, the slot becomes the max over every rank r touching g of
 *   max(1e-7, max_d max(RN(maxK[r,g,d] - m[d]), RN(m[d] - minK[r,g,d]))).
 * gathered: [P,B,H,2,2,D] in rank order.  mean NULL means +0 (raw Q). */
void ora_derive_k_boundary_amax(float* grouped, const float* gathered, const uint16_t* mean,
                                int dtype, int64_t B, int64_t H, int64_t D, int64_t rank,
                                int64_t L, int64_t P) {
    int64_t slots = ora_slots(L);
    for (int e = 0; e < 2; e++) {
        int64_t g = e == 0 ? first_group(rank, L) : last_group(rank, L);
        for (int64_t b = 0; b < B; b++)
            for (int64_t hh = 0; hh < H; hh++) {
                float best = -INFINITY;
                for (int64_t r = 0; r < P; r++) {
                    int64_t lo = r * L, hi = r * L + L;
                    int touches = lo < ORA_GROUP * g + ORA_GROUP && ORA_GROUP * g < hi;
                    if (!touches) continue;
                    int er = (g == first_group(r, L)) ? 0 : 1;
                    float c = -INFINITY;
                    for (int64_t d = 0; d < D; d++) {
                        float m = mean ? elem(mean, (b * H + hh) * D + d, dtype) : 0.0f;
                        float mn = gathered[((((r * B + b) * H + hh) * 2 + er) * 2 + 0) * D + d];
                        float mx = gathered[((((r * B + b) * H + hh) * 2 + er) * 2 + 1) * D + d];
                        c = fmaxf(c, fmaxf(mx - m, m - mn));
                    }
                    c = fmaxf(ORA_FLOOR, c);
                    best = fmaxf(best, c);
                }
                grouped[(b * H + hh) * slots + (g - first_group(rank, L))] = best;
            }
    }
}

/* ------------------------------------------------------------------ step 4: pack */

/* Quantize this rank's shard and write one chunk per destination p at send + p*stride.
 * q_amax, k_amax: [B,H,slots(L)] after derive.  mean: [B,H,D] (K is centered by it).
 * v_scale: [B,H,D] binary32 divisor of V before the E4M3 conversion, or NULL (unscaled). */
void ora_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* mean,
              int dtype, const float* q_amax, const float* k_amax, const float* v_scale,
              int64_t B, int64_t L, int64_t H, int64_t D, int64_t rank, int64_t P,
              uint8_t* send, int64_t stride) {
    int64_t h = H / P;
    int64_t slots = ora_slots(L);
    int64_t sec = align256(B * L * h * D);
    int64_t ssec = align256(4 * B * h * slots);
    int64_t g0 = first_group(rank, L);
    for (int64_t p = 0; p < P; p++) {
        uint8_t* chunk = send + p * stride;
        memset(chunk, 0, (size_t)ora_chunk_bytes(B, L, h, D));
        int8_t* q8 = (int8_t*)(chunk);
        int8_t* k8 = (int8_t*)(chunk + sec);
        uint8_t* v8 = chunk + 2 * sec;
        float* qs = (float*)(chunk + 3 * sec);
        float* ks = (float*)(chunk + 3 * sec + ssec);
        for (int64_t b = 0; b < B; b++)
            for (int64_t j = 0; j < h; j++) {
                int64_t hh = p * h + j;
                for (int64_t sl = 0; sl < slots; sl++) {
                    qs[(b * h + j) * slots + sl] = q_amax[(b * H + hh) * slots + sl] / 127.0f;
                    ks[(b * h + j) * slots + sl] = k_amax[(b * H + hh) * slots + sl] / 127.0f;
                }
                for (int64_t l = 0; l < L; l++) {
                    int64_t sl = (rank * L + l) / ORA_GROUP - g0;
                    float sq = qs[(b * h + j) * slots + sl];
                    float sk = ks[(b * h + j) * slots + sl];
                    for (int64_t d = 0; d < D; d++) {
                        int64_t src = ((b * L + l) * H + hh) * D + d;
                        int64_t dst = ((b * L + l) * h + j) * D + d;
                        float kc = elem(k, src, dtype) - elem(mean, (b * H + hh) * D + d, dtype);
                        q8[dst] = ora_quant_i8(elem(q, src, dtype), sq);
                        k8[dst] = ora_quant_i8(kc, sk);
                        float vf = elem(v, src, dtype);
                        if (v_scale) vf = vf / v_scale[(b * H + hh) * D + d];
                        v8[dst] = ora_e4m3(vf);
                    }
                }
            }
    }
}

/* ------------------------------------------------------------------ step 5: unpack */

/* unpack_for_sage (description, Returns).  recv: [P, chunk_bytes] source-major.
 * scale_sequence <= 0 means None (full width).  Outputs: q8, k8 [B,S,h,D];
 * v8 [B,D,h,Spad] with Spad = ceil(S/64)*64 and a zero tail; q_scale, k_scale [B,h,W]. */
void ora_unpack_for_sage(const uint8_t* recv, int64_t B, int64_t L, int64_t h, int64_t D,
                         int64_t P, int64_t scale_sequence, int8_t* q8, int8_t* k8,
                         uint8_t* v8, float* q_scale, float* k_scale) {
    int64_t S = P * L;
    int64_t spad = (S + ORA_GROUP - 1) / ORA_GROUP * ORA_GROUP;
    int64_t ns = scale_sequence > 0 ? scale_sequence : S;
    int64_t W = (ns + ORA_GROUP - 1) / ORA_GROUP;
    int64_t slots = ora_slots(L);
    int64_t cb = ora_chunk_bytes(B, L, h, D);
    int64_t sec = align256(B * L * h * D);
    int64_t ssec = align256(4 * B * h * slots);
    for (int64_t b = 0; b < B; b++)
        for (int64_t t = 0; t < spad; t++)
            for (int64_t j = 0; j < h; j++)
                for (int64_t d = 0; d < D; d++) {
                    uint8_t vb = 0;
                    if (t < S) {
                        const uint8_t* chunk = recv + (t / L) * cb;
                        int64_t src = ((b * L + t % L) * h + j) * D + d;
                        q8[((b * S + t) * h + j) * D + d] = (int8_t)chunk[src];
                        k8[((b * S + t) * h + j) * D + d] = (int8_t)chunk[sec + src];
                        vb = chunk[2 * sec + src];
                    }
                    v8[((b * D + d) * h + j) * spad + t] = vb;
                }
    for (int64_t b = 0; b < B; b++)
        for (int64_t j = 0; j < h; j++)
            for (int64_t g = 0; g < W; g++) {
                int64_t s = ORA_GROUP * g / L;        /* source holding the group's first row */
                int64_t sl = g - first_group(s, L);
                const uint8_t* chunk = recv + s * cb;
                float qv, kv;
                memcpy(&qv, chunk + 3 * sec + 4 * ((b * h + j) * slots + sl), 4);
                memcpy(&kv, chunk + 3 * sec + ssec + 4 * ((b * h + j) * slots + sl), 4);
                q_scale[(b * h + j) * W + g] = qv;
                k_scale[(b * h + j) * W + g] = kv;
            }
}

/* ------------------------------------------------------------------ the global K mean */

/* binary32 -> bfloat16 bits, round to nearest even (finite inputs). */
uint16_t ora_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* binary32 -> IEEE binary16 bits, round to nearest even, overflow to infinity, gradual
 * underflow (finite inputs).  Written from the format: 5 exponent bits (bias 15),
 * 10 fraction bits, subnormal step 2^-24. */
uint16_t ora_fp16_bits(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    float a = fabsf(f);
    if (a >= 65520.0f) return sign | 0x7C00;          /* rounds past the largest, 65504 */
    if (a < 0x1p-14f) {                               /* subnormal range (and zero) */
        float n = rintf(ldexpf(a, 24));               /* multiples of 2^-24; 1024 -> 2^-14 */
        return sign | (uint16_t)n;
    }
    int e2;
    frexpf(a, &e2);                                   /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    float n = rintf(ldexpf(a, 10 - E));               /* in [1024, 2048] */
    if (n == 2048.0f) {
        E += 1;
        n = 1024.0f;
    }
    return sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024));
}

/* The global K mean over the live rows [0, used) of the stacked shards k [P,B,L,H,D]:
 * a binary64 sum in row order, divided by used in binary64, rounded to binary32
 * (mean_f32 [B,H,D]) and from there to the input dtype (mean_dt [B,H,D], 16-bit patterns). */
void ora_k_mean(const uint16_t* k, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
                int64_t P, int64_t used, float* mean_f32, uint16_t* mean_dt) {
    int64_t S = P * L;
    int64_t u = used > 0 ? used : S;
    for (int64_t b = 0; b < B; b++)
        for (int64_t hh = 0; hh < H; hh++)
            for (int64_t d = 0; d < D; d++) {
                double sum = 0.0;
                for (int64_t t = 0; t < u; t++) {
                    int64_t r = t / L, l = t % L;
                    sum += (double)elem(k, (((r * B + b) * L + l) * H + hh) * D + d, dtype);
                }
                float m = (float)(sum / (double)u);
                mean_f32[(b * H + hh) * D + d] = m;
                mean_dt[(b * H + hh) * D + d] = dtype == ORA_BF16 ? ora_bf16_bits(m)
                                                                  : ora_fp16_bits(m);
            }
}
