/*
 * Seeded synthetic inputs for exact attention: counter-based random numbers
 * rounded to fp16 / bf16.  This file holds no attention arithmetic; it only
 * draws the numbers that both the FP64 checker and the GPU library are fed.
 *
 * Generator: Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3.3:
 * each round multiplies two of the four 32-bit words by fixed odd constants,
 * keeps the high halves XORed with the other two words and the round key, and
 * the two-word key is bumped by the Weyl constants between rounds.
 *
 * Element e of a tensor uses the Philox block with counter (e/2, 0, 0, 0)
 * and key (seed, tensor_id).  The four output words become two uniforms with
 * 53 random bits each; Box-Muller (Box and Muller, 1958) turns the pair into
 * two independent standard normals, and element e takes the cosine branch when
 * e is even and the sine branch when e is odd.  A uniform element takes the
 * first uniform of its block when e is even and the second when e is odd.
 * Every value is computed in double, rounded to binary32 (round to nearest
 * even) and then to the target 16-bit format (round to nearest even).  The
 * result depends only on (seed, tensor_id, e), never on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 53-bit uniform in the open interval (0, 1): (k + 1/2) * 2^-53. */
static double uniform53(uint32_t a, uint32_t b) {
    uint64_t k = ((uint64_t)a << 21) ^ (uint64_t)(b >> 11);
    return ((double)k + 0.5) * (1.0 / 9007199254740992.0);
}

/* binary32 -> binary16 bits, round to nearest even, with subnormals, inf, nan. */
uint16_t synth_f32_to_f16_bits(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (exp == 0xFFu) {
        return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    }
    int32_t e = (int32_t)exp - 127 + 15;
    if (e >= 0x1F) return (uint16_t)(sign | 0x7C00u);
    if (e <= 0) {
        /* subnormal half (or zero): value = man_full * 2^(exp-150); target unit 2^-24 */
        if (e < -10) return (uint16_t)sign;
        uint32_t full = man | 0x800000u;
        int shift = 14 - e; /* 14..24 */
        uint32_t q = full >> shift;
        uint32_t rem = full & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q += 1u;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1u; /* may carry into inf: correct */
    return (uint16_t)(sign | q);
}

/* binary32 -> bfloat16 bits, round to nearest even; nan stays nan. */
uint16_t synth_f32_to_bf16_bits(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

enum { SYNTH_NORMAL = 0, SYNTH_UNIFORM = 1 };
enum { SYNTH_F16 = 0, SYNTH_BF16 = 1, SYNTH_F32 = 2, SYNTH_F64 = 3 };

typedef struct {
    void* dst;
    int64_t begin, end;   /* element range [begin, end) of this worker, relative to element_offset */
    int64_t element_offset;
    int dist, dtype;
    double a, b;          /* normal: mean a, std b; uniform: [a, b) */
    uint32_t seed, tensor_id;
} synth_job;

static double draw(const synth_job* j, int64_t e) {
    uint32_t ctr[4] = {(uint32_t)((uint64_t)e >> 1), (uint32_t)((uint64_t)e >> 33), 0u, 0u};
    uint32_t key[2] = {j->seed, j->tensor_id};
    uint32_t r[4];
    synth_philox4x32_10(ctr, key, r);
    double u1 = uniform53(r[0], r[1]);
    double u2 = uniform53(r[2], r[3]);
    if (j->dist == SYNTH_UNIFORM) {
        double u = (e & 1) ? u2 : u1;
        return j->a + (j->b - j->a) * u;
    }
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925286766559 * u2;
    double z = (e & 1) ? rad * sin(ang) : rad * cos(ang);
    return j->a + j->b * z;
}

static void* worker(void* arg) {
    const synth_job* j = (const synth_job*)arg;
    for (int64_t i = j->begin; i < j->end; ++i) {
        double x = draw(j, j->element_offset + i);
        float f = (float)x;
        switch (j->dtype) {
            case SYNTH_F16: ((uint16_t*)j->dst)[i] = synth_f32_to_f16_bits(f); break;
            case SYNTH_BF16: ((uint16_t*)j->dst)[i] = synth_f32_to_bf16_bits(f); break;
            case SYNTH_F32: ((float*)j->dst)[i] = f; break;
            default: ((double*)j->dst)[i] = x; break;
        }
    }
    return NULL;
}

/* Fill dst[0..n) with elements element_offset .. element_offset+n-1 of the
 * stream (seed, tensor_id).  Returns 0 on success. */
int synth_fill(void* dst, int64_t n, int64_t element_offset, int dist, int dtype, double a, double b,
               uint32_t seed, uint32_t tensor_id, int nthreads) {
    if (n < 0 || !dst || nthreads < 1) return -1;
    if (nthreads > 256) nthreads = 256;
    if (n < 65536) nthreads = 1;
    pthread_t th[256];
    synth_job jobs[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        synth_job* j = &jobs[t];
        j->dst = dst; j->element_offset = element_offset; j->dist = dist; j->dtype = dtype;
        j->a = a; j->b = b; j->seed = seed; j->tensor_id = tensor_id;
        j->begin = (int64_t)t * per;
        j->end = j->begin + per < n ? j->begin + per : n;
        if (j->begin >= j->end) break;
        if (nthreads == 1) {
            worker(j);
            return 0;
        }
        if (pthread_create(&th[t], NULL, worker, j) != 0) {
            worker(j);
            continue;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* Raw Philox words for a block range, for ranking draws (sampling without replacement). */
void synth_raw_u32(uint32_t* dst, int64_t n, uint32_t seed, uint32_t tensor_id) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t ctr[4] = {(uint32_t)((uint64_t)i), (uint32_t)((uint64_t)i >> 32), 0u, 0u};
        uint32_t key[2] = {seed, tensor_id};
        uint32_t r[4];
        synth_philox4x32_10(ctr, key, r);
        dst[i] = r[0];
    }
}
