// MoE expert operation of a speculative-decoding verification pass on gfx950.
//
// What is computed (Lan, arXiv:2610.34440, Section 1): for a pass of n tokens,
// each routed to m of N experts,
//     y_t = sum_j w_tj W_down[e_tj] ( silu(W_gate[e_tj] x_t) * (W_up[e_tj] x_t) ).
// Two kernels compute it: per-slot (one expert read per slot) and deduplicating
// (the pass's slots grouped by expert, one read per distinct expert).
//
// Design for CDNA4 (this is a skinny GEMM: 1..64 token columns against expert
// weight rows streamed from HBM, about 1..g flop per weight byte):
//   * one "unit" is a slot (per-slot) or a distinct expert with its group of g
//     slots (deduplicating).  Work items are (unit, 16-row tile of the output).
//   * a workgroup of 4 wave64s owns one item; the waves split the contraction
//     dimension K in four contiguous ranges and reduce through LDS in a fixed
//     order.  Each lane issues 16-byte loads of weight rows; a wave's load covers
//     16 rows x 64 contiguous bytes, so two consecutive steps fill whole 128-byte
//     lines.
//   * the contraction runs on MFMA: the weight tile (16 rows x 32 k, bf16) is the
//     A operand straight from the load registers; the token activations (x, or
//     the hidden h) are the B operand, 16 tokens per tile, read from L2.  No
//     cross-lane reduction is needed inside a wave.  Token columns beyond the
//     group are zero and their outputs are dropped.
//   * the hidden activation h (fp32) is stored as a bf16 pair hi + lo (h ~= hi +
//     lo to 2^-17 relative) so the down projection runs on bf16 MFMA with two
//     products per step; fp32 layers use the fp32 MFMA.
//   * phase 1 (gate/up) writes h per slot; phase 2 (down) writes each slot's
//     expert output O per slot; a combine kernel forms y_t = sum_j w_tj O_tj in
//     increasing j.  Per-slot and deduplicating runs share phases 2's arithmetic
//     per token and the combine, so their results are bitwise equal.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "moe_expert.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kWaves = 4;     // waves per workgroup (split of K)
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;     // output rows per item = MFMA M
constexpr int kPerSlot = 0, kDedup = 1;

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// bf16 16x16x32 MFMA: D += A(16x32) B(32x16).  Lane l supplies A row l%16 and B
// column l%16, elements k = 8*(l/16) .. +8 of the step (any k permutation that A
// and B share gives the same sum).
__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32: four 16x16x4 MFMAs; lane group q = l/16 holds 4 consecutive k of the
// 16-wide step, MFMA i takes element i of every group.
__device__ __forceinline__ f32x4 mma_f32(u32x4 a, u32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
}

template <bool BF16>
struct Fmt {
    static constexpr int kEsize = BF16 ? 2 : 4;
    static constexpr int kPer = 16 / kEsize;     // elements per 16-byte lane load
    static constexpr int kStep = 4 * kPer;       // k covered by one wave step
    __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) { return BF16 ? mma_bf16(a, b, c) : mma_f32(a, b, c); }
};

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

struct Route {
    const int32_t* ids;       // [n*m]
    const int32_t* offset;    // dedup: [N+1]
    const int32_t* sbe;       // dedup: [n*m]
    const int32_t* distinct;  // dedup: [N]
    const int32_t* u_err;     // dedup: [2]
    int32_t n, m, N;
};

// Resolve a unit to its expert and slot group.  Returns false when the unit
// holds no work (past U, or an invalid id).  Uniform across the workgroup.
template <int MODE>
__device__ __forceinline__ bool resolve(const Route& r, int unit, int& e, int& beg, int& g) {
    if (MODE == kPerSlot) {
        if (unit >= r.n * r.m) return false;
        e = r.ids[unit];
        if (e < 0 || e >= r.N) return false;
        beg = unit;
        g = 1;
        return true;
    } else {
        const int U = r.u_err[0];
        if (unit >= U) return false;
        e = r.distinct[unit];
        if (e < 0 || e >= r.N) return false;
        beg = r.offset[e];
        g = r.offset[e + 1] - beg;
        // a group lies inside the n*m slot list; anything else is not a
        // moe_route_group output and is skipped rather than read out of bounds
        return g > 0 && beg >= 0 && beg + g <= r.n * r.m;
    }
}

template <int MODE>
__device__ __forceinline__ int member_slot(const Route& r, int beg, int gi) {
    if (MODE == kPerSlot) return beg;
    const int s = r.sbe[beg + gi];
    return (s >= 0 && s < r.n * r.m) ? s : 0;
}

// ---------------------------------------------------------------------------
// Grouping: histogram, exclusive scan and stable scatter of slot indices by
// expert id, in one workgroup of 256 threads (n*m <= 256, N <= 1024).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_route_group(const int32_t* __restrict__ ids, int n, int m, int N,
                                                     int32_t* __restrict__ count, int32_t* __restrict__ offset,
                                                     int32_t* __restrict__ sbe, int32_t* __restrict__ distinct,
                                                     int32_t* __restrict__ u_err) {
    __shared__ int s_ids[MOE_MAX_SLOTS];
    __shared__ int s_cnt[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS];
    __shared__ int s_dpos[MOE_MAX_EXPERTS];
    __shared__ int s_part[256][2];
    __shared__ int s_flag;
    const int tid = threadIdx.x;
    const int nm = n * m;
    for (int e = tid; e < N; e += 256) s_cnt[e] = 0;
    if (tid == 0) s_flag = 0;
    const int id = tid < nm ? ids[tid] : -1;
    const bool valid = tid < nm && id >= 0 && id < N;
    s_ids[tid] = valid ? id : -1;
    __syncthreads();
    if (tid < nm) {
        if (!valid) {
            atomicOr(&s_flag, 1);
        } else {
            const int t = tid / m, j = tid - t * m;
            for (int jj = 0; jj < j; ++jj)
                if (s_ids[t * m + jj] == id) atomicOr(&s_flag, 1);
            atomicAdd(&s_cnt[id], 1);
        }
    }
    __syncthreads();
    // exclusive scan of counts and of presence over N entries: each thread owns
    // a contiguous chunk, then a Hillis-Steele scan of the 256 chunk totals.
    const int chunk = (N + 255) / 256;
    const int e0 = tid * chunk;
    int sc = 0, sp = 0;
    for (int e = e0; e < e0 + chunk && e < N; ++e) {
        sc += s_cnt[e];
        sp += s_cnt[e] > 0;
    }
    s_part[tid][0] = sc;
    s_part[tid][1] = sp;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        int a0 = 0, a1 = 0;
        if (tid >= d) {
            a0 = s_part[tid - d][0];
            a1 = s_part[tid - d][1];
        }
        __syncthreads();
        s_part[tid][0] += a0;
        s_part[tid][1] += a1;
        __syncthreads();
    }
    int run_c = s_part[tid][0] - sc, run_p = s_part[tid][1] - sp;  // exclusive
    for (int e = e0; e < e0 + chunk && e < N; ++e) {
        s_off[e] = run_c;
        s_dpos[e] = run_p;
        run_c += s_cnt[e];
        run_p += s_cnt[e] > 0;
    }
    __syncthreads();
    const int total = s_part[255][0];
    const int U = s_part[255][1];
    for (int e = tid; e < N; e += 256) {
        count[e] = s_cnt[e];
        offset[e] = s_off[e];
        if (s_cnt[e] > 0) distinct[s_dpos[e]] = e;  // positions 0 .. U-1
        if (e >= U) distinct[e] = -1;               // positions U .. N-1
    }
    if (tid == 0) offset[N] = total;
    if (tid < nm) {
        if (valid) {
            int rank = 0;
            for (int s = 0; s < tid; ++s) rank += (s_ids[s] == id);
            sbe[s_off[id] + rank] = tid;
        }
        if (tid >= total) sbe[tid] = -1;
    }
    if (tid == 0) {
        u_err[0] = U;
        u_err[1] = s_flag ? MOE_E_IDS : MOE_OK;
    }
}

// ---------------------------------------------------------------------------
// Phase 1: gate and up projections of a unit's tokens for 16 rows of d_ff,
// h = silu(W_gate x) * (W_up x).  bf16 layers store h as hi/lo bf16 pairs
// (hi at h, lo at h + nm*d_ff), fp32 layers as fp32.
// ---------------------------------------------------------------------------
template <bool BF16, int MODE, int NT, int UNROLL>
__global__ __launch_bounds__(kThreads) void k_gate_up(const void* __restrict__ wg_, const void* __restrict__ wu_,
                                                      const void* __restrict__ x_, Route r, void* __restrict__ h_,
                                                      int d, int d_ff, int ntiles) {
    using F = Fmt<BF16>;
    __shared__ f32x4 red[kWaves][2][NT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int unit = blockIdx.x / ntiles, rt = blockIdx.x - unit * ntiles;
    int e, beg, g;
    if (!resolve<MODE>(r, unit, e, beg, g)) return;
    const int lr = lane & 15, q = lane >> 4;
    const int row = rt * kTile + lr;
    const bool row_ok = row < d_ff;
    const char* wg = reinterpret_cast<const char*>(wg_) + ((size_t)e * d_ff + (row_ok ? row : 0)) * d * F::kEsize;
    const char* wu = reinterpret_cast<const char*>(wu_) + ((size_t)e * d_ff + (row_ok ? row : 0)) * d * F::kEsize;
    const int nsteps = (d + F::kStep - 1) / F::kStep;
    const int s0 = wave * nsteps / kWaves, s1 = (wave + 1) * nsteps / kWaves;
    const int nm = r.n * r.m;

    for (int base = 0; base < g; base += 16 * NT) {
        const char* xrow[NT];
        bool tok_ok[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int gi = base + tt * 16 + lr;
            tok_ok[tt] = gi < g;
            const int slot = tok_ok[tt] ? member_slot<MODE>(r, beg, gi) : 0;
            xrow[tt] = reinterpret_cast<const char*>(x_) + (size_t)(slot / r.m) * d * F::kEsize;
        }
        f32x4 accg[NT], accu[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            accg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int s = s0; s < s1; s += UNROLL) {
            u32x4 ag[UNROLL], au[UNROLL], bx[UNROLL][NT];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int k = (s + u) * F::kStep + q * F::kPer;
                const bool kin = (s + u < s1) && (k < d);
                const size_t off = (size_t)k * F::kEsize;
                ag[u] = (kin && row_ok) ? ld16(wg + off) : zero4();
                au[u] = (kin && row_ok) ? ld16(wu + off) : zero4();
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) bx[u][tt] = (kin && tok_ok[tt]) ? ld16(xrow[tt] + off) : zero4();
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    accg[tt] = F::mma(ag[u], bx[u][tt], accg[tt]);
                    accu[tt] = F::mma(au[u], bx[u][tt], accu[tt]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            red[wave][0][tt][lane] = accg[tt];
            red[wave][1][tt][lane] = accu[tt];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 G = red[0][0][tt][lane], Uu = red[0][1][tt][lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) {
                    G += red[w][0][tt][lane];
                    Uu += red[w][1][tt][lane];
                }
                const int gi = base + tt * 16 + lr;  // output column = lane % 16
                if (gi < g) {
                    const int slot = member_slot<MODE>(r, beg, gi);
                    const int f0 = rt * kTile + 4 * q;  // output rows 4q .. 4q+3
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = f0 + i;
                        if (f < d_ff) {
                            const float hv = silu(G[i]) * Uu[i];
                            const size_t idx = (size_t)slot * d_ff + f;
                            if (BF16) {
                                const uint16_t hi = bf16_rne(hv);
                                const uint16_t lo = bf16_rne(hv - bf16_to_f32(hi));
                                reinterpret_cast<uint16_t*>(h_)[idx] = hi;
                                reinterpret_cast<uint16_t*>(h_)[(size_t)nm * d_ff + idx] = lo;
                            } else {
                                reinterpret_cast<float*>(h_)[idx] = hv;
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Phase 2: down projection of a unit's h for 16 rows of d_model; writes the
// expert output O[slot][row] (fp32) of every slot of the unit.
// ---------------------------------------------------------------------------
template <bool BF16, int MODE, int NT, int UNROLL>
__global__ __launch_bounds__(kThreads) void k_down(const void* __restrict__ wd_, const void* __restrict__ h_, Route r,
                                                   float* __restrict__ O, int d, int d_ff, int ntiles) {
    using F = Fmt<BF16>;
    __shared__ f32x4 red[kWaves][NT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int unit = blockIdx.x / ntiles, rt = blockIdx.x - unit * ntiles;
    int e, beg, g;
    if (!resolve<MODE>(r, unit, e, beg, g)) return;
    const int lr = lane & 15, q = lane >> 4;
    const int row = rt * kTile + lr;
    const bool row_ok = row < d;
    const char* wd = reinterpret_cast<const char*>(wd_) + ((size_t)e * d + (row_ok ? row : 0)) * d_ff * F::kEsize;
    const int nsteps = (d_ff + F::kStep - 1) / F::kStep;
    const int s0 = wave * nsteps / kWaves, s1 = (wave + 1) * nsteps / kWaves;
    const int nm = r.n * r.m;
    const char* hbase = reinterpret_cast<const char*>(h_);
    const size_t lo_off = (size_t)nm * d_ff * 2;  // bf16: lo half after hi half

    for (int base = 0; base < g; base += 16 * NT) {
        const char* hrow[NT];
        bool tok_ok[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int gi = base + tt * 16 + lr;
            tok_ok[tt] = gi < g;
            const int slot = tok_ok[tt] ? member_slot<MODE>(r, beg, gi) : 0;
            hrow[tt] = hbase + (size_t)slot * d_ff * F::kEsize;
        }
        f32x4 acc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = s0; s < s1; s += UNROLL) {
            u32x4 a[UNROLL], bh[UNROLL][NT], bl[UNROLL][NT];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int k = (s + u) * F::kStep + q * F::kPer;
                const bool kin = (s + u < s1) && (k < d_ff);
                const size_t off = (size_t)k * F::kEsize;
                a[u] = (kin && row_ok) ? ld16(wd + off) : zero4();
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    bh[u][tt] = (kin && tok_ok[tt]) ? ld16(hrow[tt] + off) : zero4();
                    if (BF16) bl[u][tt] = (kin && tok_ok[tt]) ? ld16(hrow[tt] + lo_off + off) : zero4();
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    acc[tt] = F::mma(a[u], bh[u][tt], acc[tt]);
                    if (BF16) acc[tt] = F::mma(a[u], bl[u][tt], acc[tt]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) red[wave][tt][lane] = acc[tt];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 v = red[0][tt][lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) v += red[w][tt][lane];
                const int gi = base + tt * 16 + lr;
                if (gi < g) {
                    const int slot = member_slot<MODE>(r, beg, gi);
                    const int i0 = rt * kTile + 4 * q;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (i0 + i < d) O[(size_t)slot * d + i0 + i] = v[i];
                }
            }
        }
        __syncthreads();
    }
}

// y[t][i] (+)= sum_{j ascending, valid id} w[t][j] * O[t*m+j][i]
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ O, const int32_t* __restrict__ ids,
                                                 const float* __restrict__ w, float* __restrict__ y, int n, int m,
                                                 int N, int d, int accumulate) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n * d) return;
    const int t = idx / d, i = idx - t * d;
    float acc = 0.f;
    for (int j = 0; j < m; ++j) {
        const int s = t * m + j;
        const int e = ids[s];
        if (e >= 0 && e < N) acc = fmaf(w[s], O[(size_t)s * d + i], acc);
    }
    y[idx] = accumulate ? y[idx] + acc : acc;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const moe_layer_desc* d, int32_t n) {
    if (!d) return MOE_E_INVAL;
    if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_E_DTYPE;
    if (d->d_model < 8 || d->d_ff < 8 || (d->d_model % 8) || (d->d_ff % 8)) return MOE_E_DTYPE;
    if (d->N < 1 || d->N > MOE_MAX_EXPERTS || d->m < 1 || d->m > d->N) return MOE_E_INVAL;
    if (n < 1 || n > MOE_MAX_TOKENS || (int64_t)n * d->m > MOE_MAX_SLOTS) return MOE_E_INVAL;
    if (d->flags & ~MOE_FLAG_ACCUMULATE) return MOE_E_INVAL;
    return MOE_OK;
}

struct Ws {
    void* h;
    float* O;
};

size_t ws_bytes_for(const moe_layer_desc* d, int32_t n) {
    const size_t nm = (size_t)n * d->m;
    return align_up(nm * d->d_ff * 4) + align_up(nm * d->d_model * 4);
}

Ws carve(const moe_layer_desc* d, int32_t n, void* ws) {
    const size_t nm = (size_t)n * d->m;
    Ws w;
    w.h = ws;
    w.O = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up(nm * d->d_ff * 4));
    return w;
}

int token_tiles(int32_t n) { return n <= 16 ? 1 : (n <= 32 ? 2 : 4); }

template <bool BF16, int MODE, int NT>
void launch_phases(const moe_layer_desc* d, const moe_layer_weights* W, const void* x, const Route& r, int units,
                   const Ws& ws, hipStream_t st, hipEvent_t* ev, int& evi) {
    constexpr int U1 = NT == 1 ? 8 : (NT == 2 ? 4 : 2);
    constexpr int U2 = NT == 1 ? 8 : (NT == 2 ? 4 : 2);
    const int t1 = (d->d_ff + kTile - 1) / kTile;
    const int t2 = (d->d_model + kTile - 1) / kTile;
    hipLaunchKernelGGL((k_gate_up<BF16, MODE, NT, U1>), dim3(units * t1), dim3(kThreads), 0, st, W->w_gate,
                       W->w_up, x, r, ws.h, d->d_model, d->d_ff, t1);
    if (ev) (void)hipEventRecord(ev[evi++], st);
    hipLaunchKernelGGL((k_down<BF16, MODE, NT, U2>), dim3(units * t2), dim3(kThreads), 0, st, W->w_down, ws.h, r,
                       ws.O, d->d_model, d->d_ff, t2);
    if (ev) (void)hipEventRecord(ev[evi++], st);
}

template <int MODE>
int run_expert(const moe_layer_desc* d, const moe_layer_weights* W, const void* x, const int32_t* ids,
               const float* w, int32_t n, const int32_t* offset, const int32_t* sbe, const int32_t* distinct,
               const int32_t* u_err, float* y, void* ws, size_t ws_bytes, void* stream, void* const* events,
               int32_t n_events) {
    int rc = check_desc(d, n);
    if (rc != MOE_OK) return rc;
    if (!W || !W->w_gate || !W->w_up || !W->w_down || !x || !ids || !w || !y || !ws) return MOE_E_INVAL;
    if (MODE == kDedup && (!offset || !sbe || !distinct || !u_err)) return MOE_E_INVAL;
    if (!aligned16(W->w_gate) || !aligned16(W->w_up) || !aligned16(W->w_down) || !aligned16(x))
        return MOE_E_INVAL;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_E_INVAL;
    if (ws_bytes < ws_bytes_for(d, n)) return MOE_E_WORKSPACE;
    if (events) {
        if (n_events != 4) return MOE_E_INVAL;
        for (int i = 0; i < n_events; ++i)
            if (!events[i]) return MOE_E_INVAL;
    } else if (n_events != 0) {
        return MOE_E_INVAL;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipEvent_t* ev = events ? reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)) : nullptr;
    int evi = 0;
    Route r{ids, offset, sbe, distinct, u_err, n, d->m, d->N};
    const Ws wsp = carve(d, n, ws);
    const int nm = n * d->m;
    const int units = MODE == kPerSlot ? nm : (nm < d->N ? nm : d->N);
    (void)hipGetLastError();
    if (ev) (void)hipEventRecord(ev[evi++], st);
    const bool bf = d->dtype == MOE_BF16;
    const int nt = MODE == kPerSlot ? 1 : token_tiles(n);
    if (bf) {
        if (nt == 1) launch_phases<true, MODE, 1>(d, W, x, r, units, wsp, st, ev, evi);
        else if (nt == 2) launch_phases<true, MODE, 2>(d, W, x, r, units, wsp, st, ev, evi);
        else launch_phases<true, MODE, 4>(d, W, x, r, units, wsp, st, ev, evi);
    } else {
        if (nt == 1) launch_phases<false, MODE, 1>(d, W, x, r, units, wsp, st, ev, evi);
        else if (nt == 2) launch_phases<false, MODE, 2>(d, W, x, r, units, wsp, st, ev, evi);
        else launch_phases<false, MODE, 4>(d, W, x, r, units, wsp, st, ev, evi);
    }
    const int nd = n * d->d_model;
    hipLaunchKernelGGL(k_combine, dim3((nd + 255) / 256), dim3(256), 0, st, wsp.O, ids, w, y, n, d->m, d->N,
                       d->d_model, (d->flags & MOE_FLAG_ACCUMULATE) ? 1 : 0);
    if (ev) (void)hipEventRecord(ev[evi++], st);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace

extern "C" {

int moe_route_group(const int32_t* ids, int32_t n, int32_t m, int32_t N, int32_t* count, int32_t* offset,
                    int32_t* slot_by_expert, int32_t* distinct, int32_t* u_and_err, void* hip_stream) {
    if (!ids || !count || !offset || !slot_by_expert || !distinct || !u_and_err) return MOE_E_INVAL;
    if (N < 1 || N > MOE_MAX_EXPERTS || m < 1 || m > N || n < 1 || (int64_t)n * m > MOE_MAX_SLOTS)
        return MOE_E_INVAL;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_route_group, dim3(1), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream), ids, n, m, N,
                       count, offset, slot_by_expert, distinct, u_and_err);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

size_t moe_workspace_bytes(const moe_layer_desc* desc, int32_t n, int32_t kind) {
    if (kind != MOE_KIND_SLOT && kind != MOE_KIND_DEDUP) return 0;
    if (check_desc(desc, n) != MOE_OK) return 0;
    return ws_bytes_for(desc, n);
}

int moe_kernels_per_call(int32_t kind) {
    if (kind != MOE_KIND_SLOT && kind != MOE_KIND_DEDUP) return MOE_E_INVAL;
    return 3;
}

int moe_expert_perslot(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                       const int32_t* ids, const float* w, int32_t n, float* y, void* ws, size_t ws_bytes,
                       void* hip_stream) {
    return run_expert<kPerSlot>(desc, weights, x, ids, w, n, nullptr, nullptr, nullptr, nullptr, y, ws, ws_bytes,
                                hip_stream, nullptr, 0);
}

int moe_expert_dedup(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                     const int32_t* ids, const float* w, int32_t n, const int32_t* offset,
                     const int32_t* slot_by_expert, const int32_t* distinct, const int32_t* u_and_err, float* y,
                     void* ws, size_t ws_bytes, void* hip_stream) {
    return run_expert<kDedup>(desc, weights, x, ids, w, n, offset, slot_by_expert, distinct, u_and_err, y, ws,
                              ws_bytes, hip_stream, nullptr, 0);
}

int moe_expert_perslot_ev(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                          const int32_t* ids, const float* w, int32_t n, float* y, void* ws, size_t ws_bytes,
                          void* hip_stream, void* const* events, int32_t n_events) {
    if (!events) return MOE_E_INVAL;
    return run_expert<kPerSlot>(desc, weights, x, ids, w, n, nullptr, nullptr, nullptr, nullptr, y, ws, ws_bytes,
                                hip_stream, events, n_events);
}

int moe_expert_dedup_ev(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                        const int32_t* ids, const float* w, int32_t n, const int32_t* offset,
                        const int32_t* slot_by_expert, const int32_t* distinct, const int32_t* u_and_err,
                        float* y, void* ws, size_t ws_bytes, void* hip_stream, void* const* events,
                        int32_t n_events) {
    if (!events) return MOE_E_INVAL;
    return run_expert<kDedup>(desc, weights, x, ids, w, n, offset, slot_by_expert, distinct, u_and_err, y, ws,
                              ws_bytes, hip_stream, events, n_events);
}

}  // extern "C"
