/*
 * Seeded synthetic inputs: counter-based normal deviates, rounded to fp32 or
 * bf16.  This library holds no arithmetic of the MoE expert operation; it only
 * produces the weight and activation values that both the GPU path and the CPU
 * oracle consume.
 *
 * Generator (random access by element index, so any expert of any layer can be
 * regenerated on its own):
 *   x_i = SplitMix64 output number i of the stream whose state starts at `key`,
 *         i.e. mix64(key + (i + 1) * 0x9E3779B97F4A7C15)   (Steele, Lea, Flood,
 *         "Fast splittable pseudorandom number generators", OOPSLA 2014).
 *   Normal pair p (elements 2p, 2p+1) by the Box-Muller transform in double:
 *         u1 = ((x_{2p} >> 11) + 1) * 2^-53      in (0, 1]
 *         u2 =  (x_{2p+1} >> 11)    * 2^-53      in [0, 1)
 *         r  = sqrt(-2 ln u1),  z_{2p} = r cos(2 pi u2),  z_{2p+1} = r sin(2 pi u2)
 *   Value i = sigma * z_i, rounded to nearest-even fp32, then (for bf16) the fp32
 *   bits rounded to nearest-even bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t sm_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

uint64_t synth_splitmix_at(uint64_t key, uint64_t i) { return sm_at(key, i); }

/* Normal pair p of stream `key`: z[0] = element 2p, z[1] = element 2p+1. */
static inline void normal_pair(uint64_t key, uint64_t p, double z[2]) {
    double u1 = (double)((sm_at(key, 2 * p) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(sm_at(key, 2 * p + 1) >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    z[0] = r * cos(th);
    z[1] = r * sin(th);
}

/* Elements [start, start+count) of stream `key`, scaled by sigma, written through
 * `put(j, value)` for j = 0..count-1.  Pairs are computed once each. */
#define FILL_STREAM(key, start, count, PUT)                                          \
    do {                                                                            \
        uint64_t p0 = (start) >> 1, p1 = ((start) + (uint64_t)(count) + 1) >> 1;    \
        _Pragma("omp parallel for schedule(static)")                                \
        for (int64_t pp = (int64_t)p0; pp < (int64_t)p1; ++pp) {                   \
            double z[2];                                                            \
            normal_pair((key), (uint64_t)pp, z);                                    \
            for (int h = 0; h < 2; ++h) {                                           \
                uint64_t i = 2 * (uint64_t)pp + (uint64_t)h;                        \
                if (i >= (start) && i < (start) + (uint64_t)(count)) {              \
                    int64_t j = (int64_t)(i - (start));                             \
                    PUT(j, z[h]);                                                   \
                }                                                                   \
            }                                                                       \
        }                                                                           \
    } while (0)

void synth_normal_f64(uint64_t key, uint64_t start, int64_t count, double* out) {
#define PUT_F64(j, v) out[j] = (v)
    FILL_STREAM(key, start, count, PUT_F64);
}

void synth_normal_f32(uint64_t key, uint64_t start, int64_t count, double sigma, float* out) {
#define PUT_F32(j, v) out[j] = (float)(sigma * (v))
    FILL_STREAM(key, start, count, PUT_F32);
}

void synth_normal_bf16(uint64_t key, uint64_t start, int64_t count, double sigma, uint16_t* out) {
#define PUT_BF16(j, v) out[j] = f32_to_bf16_rne((float)(sigma * (v)))
    FILL_STREAM(key, start, count, PUT_BF16);
}

/* Fill `n_blocks` consecutive blocks of `block` elements, block b being elements
 * [0, block) of stream keys[b] (one block per expert of a weight tensor). */
void synth_blocks_bf16(const uint64_t* keys, int64_t n_blocks, int64_t block, double sigma,
                       uint16_t* out) {
    for (int64_t b = 0; b < n_blocks; ++b) synth_normal_bf16(keys[b], 0, block, sigma, out + b * block);
}

void synth_blocks_f32(const uint64_t* keys, int64_t n_blocks, int64_t block, double sigma,
                      float* out) {
    for (int64_t b = 0; b < n_blocks; ++b) synth_normal_f32(keys[b], 0, block, sigma, out + b * block);
}
