/*
 * synth.c - seeded, counter-based synthetic inputs for the MoE layer.
 *
 * This module only MAKES inputs (activations, weights, biases, 4-bit packed
 * weights).  It holds none of the layer's arithmetic: no sigmoid, no routing,
 * no matmul.  Both the CPU oracle and the GPU path read what it writes.
 *
 * Generator: every element i of tensor `tid` under seed `seed` is a pure
 * function of (seed, tid, i), so any element can be regenerated on its own and
 * the result does not depend on thread count or chunking.
 *   - uniform bits: the SplitMix64 output function (Steele, Lea, Flood,
 *     "Fast splittable pseudorandom number generators", OOPSLA 2014) applied
 *     to a Weyl sequence key + (counter+1) * golden-gamma;
 *   - normals: the Box-Muller transform in double precision, one pair of
 *     uniforms per pair of elements (even element -> cosine branch, odd ->
 *     sine branch);
 *   - bf16: the double is rounded to fp32, then fp32 -> bf16 with
 *     round-to-nearest-even.
 * 4-bit affine group quantisation (groups of 64 along the input axis):
 *   s = bf16((max-min)/15), b = bf16(min), q = clamp(rint((w-b)/s), 0, 15),
 *   q = 0 when s == 0; eight 4-bit codes per uint32, element i at bits 4*(i%8).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t key_of(uint64_t seed, uint64_t tid) {
    return sm_mix(sm_mix(seed * GAMMA + 0x243F6A8885A308D3ULL) + tid * GAMMA);
}

/* 64 random bits for counter c of stream `key` */
static inline uint64_t bits_at(uint64_t key, uint64_t c) { return sm_mix(key + (c + 1) * GAMMA); }

uint64_t synth_bits(uint64_t seed, uint64_t tid, uint64_t c) { return bits_at(key_of(seed, tid), c); }

/* standard normal for element i (Box-Muller on the pair i/2) */
static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    uint64_t a = bits_at(key, 2 * p), b = bits_at(key, 2 * p + 1);
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53; /* (0,1) */
    double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0,1) */
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* both normals of pair p (elements 2p and 2p+1); same values as normal_at */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    uint64_t a = bits_at(key, 2 * p), b = bits_at(key, 2 * p + 1);
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53;
    double u2 = (double)(b >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

/* out[j] = float(std * N(0,1) element (start+j)) + mean */
void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, double mean, double std,
                      float* out) {
    uint64_t key = key_of(seed, tid);
    if (n <= 0) return;
    uint64_t p0 = start >> 1, p1 = (start + (uint64_t)n - 1) >> 1;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q <= (int64_t)(p1 - p0); ++q) {
        uint64_t p = p0 + (uint64_t)q;
        double z0, z1;
        normal_pair(key, p, &z0, &z1);
        int64_t j0 = (int64_t)(2 * p) - (int64_t)start;
        if (j0 >= 0 && j0 < n) out[j0] = (float)(mean + std * z0);
        if (j0 + 1 >= 0 && j0 + 1 < n) out[j0 + 1] = (float)(mean + std * z1);
    }
}

void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, double mean, double std,
                       uint16_t* out) {
    uint64_t key = key_of(seed, tid);
    if (n <= 0) return;
    uint64_t p0 = start >> 1, p1 = (start + (uint64_t)n - 1) >> 1;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q <= (int64_t)(p1 - p0); ++q) {
        uint64_t p = p0 + (uint64_t)q;
        double z0, z1;
        normal_pair(key, p, &z0, &z1);
        int64_t j0 = (int64_t)(2 * p) - (int64_t)start;
        if (j0 >= 0 && j0 < n) out[j0] = f32_to_bf16_rne((float)(mean + std * z0));
        if (j0 + 1 >= 0 && j0 + 1 < n) out[j0 + 1] = f32_to_bf16_rne((float)(mean + std * z1));
    }
}

/* fp32 -> bf16 (RNE) conversion of an existing buffer */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}

/*
 * 4-bit affine quantisation of `rows` rows of length `cols` (cols % 64 == 0) whose fp32
 * values are the normals of tensor (seed, tid) starting at element `start`, scaled by std.
 * q:  uint32 [rows, cols/8]; s, b: bf16 [rows, cols/64].
 */
void synth_q4_normal(uint64_t seed, uint64_t tid, uint64_t start, int64_t rows, int64_t cols, double std,
                     uint32_t* q, uint16_t* s, uint16_t* b) {
    uint64_t key = key_of(seed, tid);
    int64_t ng = cols / 64;
#pragma omp parallel for schedule(static)
    for (int64_t rg = 0; rg < rows * ng; ++rg) {
        int64_t r = rg / ng, g = rg % ng;
        float w[64];
        uint64_t base = start + (uint64_t)(r * cols + g * 64);
        float mn = INFINITY, mx = -INFINITY;
        for (int i = 0; i < 64; i += 2) {
            double z0, z1; /* base is even: elements base+i, base+i+1 form one pair */
            normal_pair(key, (base + (uint64_t)i) >> 1, &z0, &z1);
            w[i] = (float)(std * z0);
            w[i + 1] = (float)(std * z1);
        }
        for (int i = 0; i < 64; ++i) {
            if (w[i] < mn) mn = w[i];
            if (w[i] > mx) mx = w[i];
        }
        uint16_t sb = f32_to_bf16_rne((mx - mn) / 15.0f);
        uint16_t bb = f32_to_bf16_rne(mn);
        float sf = bf16_to_f32(sb), bf = bf16_to_f32(bb);
        uint32_t* qw = q + r * (cols / 8) + g * 8;
        for (int k = 0; k < 8; ++k) qw[k] = 0;
        for (int i = 0; i < 64; ++i) {
            int code = 0;
            if (sf != 0.0f) {
                float v = rintf((w[i] - bf) / sf);
                code = v < 0.0f ? 0 : (v > 15.0f ? 15 : (int)v);
            }
            qw[i / 8] |= (uint32_t)code << (4 * (i % 8));
        }
        s[r * ng + g] = sb;
        b[r * ng + g] = bb;
    }
}

/* fp32 -> OCP E4M3 code, round to nearest even, magnitudes above 448 saturate to 448 (the
 * quantiser of an fp8 checkpoint; never produces NaN) */
static uint8_t e4m3_encode(float v) {
    uint8_t sg = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (!(a < 448.0f)) return (uint8_t)(sg | 0x7E);
    if (a < 0x1p-6f) {                       /* subnormal range: steps of 2^-9 */
        int m = (int)rintf(a * 512.0f);      /* exact scaling, RNE; m == 8 is the smallest normal */
        return (uint8_t)(sg | m);
    }
    int ex;
    frexpf(a, &ex);                          /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                          /* a in [2^E, 2^(E+1)) */
    int m = (int)rintf((ldexpf(a, -E) - 1.0f) * 8.0f);
    if (m == 8) { m = 0; E += 1; }
    int e = E + 7;
    if (e > 15 || (e == 15 && m == 7)) return (uint8_t)(sg | 0x7E);
    return (uint8_t)(sg | (e << 3) | m);
}

/*
 * fp8 (E4M3) quantisation with one fp32 scale per 128 x 128 block, of `nmat` stacked [rows, cols]
 * matrices whose fp32 values are the normals of tensor (seed, tid) from element `start`, scaled
 * by std (cols even).  Block scale = max |w| / 448 (1 for an all-zero block); code = E4M3 of
 * w / scale.  q: uint8 [nmat, rows, cols]; s: fp32 [nmat, ceil(rows/128), ceil(cols/128)].
 */
void synth_fp8_normal(uint64_t seed, uint64_t tid, uint64_t start, int64_t nmat, int64_t rows, int64_t cols,
                      double std, uint8_t* q, float* s) {
    uint64_t key = key_of(seed, tid);
    const int64_t nbr = (rows + 127) / 128, nbc = (cols + 127) / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nmat * nbr * nbc; ++blk) {
        const int64_t mt = blk / (nbr * nbc), br = (blk / nbc) % nbr, bc = blk % nbc;
        const int64_t r0 = br * 128, c0 = bc * 128;
        const int64_t nr = rows - r0 < 128 ? rows - r0 : 128, nc = cols - c0 < 128 ? cols - c0 : 128;
        float w[128 * 128];
        float amax = 0.0f;
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t c = 0; c < nc; c += 2) {
                const uint64_t el = start + (uint64_t)((mt * rows + r0 + r) * cols + c0 + c);
                double z0, z1; /* el is even: elements el, el+1 form one pair */
                normal_pair(key, el >> 1, &z0, &z1);
                w[r * 128 + c] = (float)(std * z0);
                w[r * 128 + c + 1] = (float)(std * z1);
                if (fabsf(w[r * 128 + c]) > amax) amax = fabsf(w[r * 128 + c]);
                if (fabsf(w[r * 128 + c + 1]) > amax) amax = fabsf(w[r * 128 + c + 1]);
            }
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t c = 0; c < nc; ++c)
                q[(mt * rows + r0 + r) * cols + c0 + c] = e4m3_encode(w[r * 128 + c] / sc);
        s[(mt * nbr + br) * nbc + bc] = sc;
    }
}

/* out[j] = uniform [0,1) double from the 53 high bits of counter start+j */
void synth_uniform_f64(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, double* out) {
    uint64_t key = key_of(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = (double)(bits_at(key, start + (uint64_t)j) >> 11) * 0x1.0p-53;
}
