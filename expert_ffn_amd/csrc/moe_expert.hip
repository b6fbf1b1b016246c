// MoE expert operation of a speculative-decoding verification pass on gfx950.
//
// What is computed (Lan, arXiv:2610.34440, Section 1): for a pass of n tokens,
// each routed to m of N experts,
//     y_t = sum_j w_tj W_down[e_tj] ( silu(W_gate[e_tj] x_t) * (W_up[e_tj] x_t) ).
// Two kernels compute it: per-slot (one expert read per slot) and deduplicating
// (the pass's slots grouped by expert, one read per distinct expert).
//
// Design for CDNA4.  The operation is a skinny GEMM (1..64 token columns against
// expert weight rows streamed from HBM, 1..g flop per weight byte), so it is
// bound by HBM bandwidth and, at small n, by fixed latency.  One launch per pass:
//   * a "unit" is a slot (per-slot) or a distinct expert with its group of slots
//     (deduplicating).  Grid = [gate/up items][down items], each item a 16-row
//     output tile of one unit, owned by a workgroup of 4 wave64s that split the
//     contraction dimension K into four contiguous ranges.
//   * the contraction runs on MFMA (bf16 16x16x32, or fp32 16x16x4): the weight
//     tile is the A operand taken straight from buffer loads (16 B per lane, row
//     lane%16, k-group lane/16); the token activations are the B operand, 16
//     token columns per tile.  Loads run in a per-wave register ring of P steps,
//     so a wave keeps P steps of operands in flight continuously.  Out-of-range
//     rows, k and token columns are buffer-descriptor misses, which return zero
//     and touch no memory.
//   * a down item first requests its W_down rows, then waits (bounded) on the
//     unit's h-ready counter, which the unit's gate/up items raise after writing
//     h.  Gate/up items have lower workgroup ids than every down item, so they are
//     dispatched first and never wait; the wait always ends.
//   * the last down item to finish a row tile (a counter per tile) combines
//     y_t = sum_j w_tj O_tj over the tile's rows in increasing j, so per-slot and
//     deduplicating results are bitwise equal.
//   * the deduplicating kernel groups the slots by expert in every workgroup's
//     prologue (n*m <= 256 ids, LDS bitmap + ballots): the same stable grouping
//     as moe_route_group, without a second launch.
//   * h (fp32) is stored as a bf16 pair hi + lo (h = hi + lo to 2^-17 relative) so
//     the down projection runs on bf16 MFMA with two products per step.
//   * the synchronisation counters live in the caller's workspace, one per
//     128-byte line; each is zeroed again by the last workgroup that uses it in
//     the launch (the combining workgroup for a tile counter, the last down item
//     of a unit for the unit's counters).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "moe_expert.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kWaves = 4;  // waves per workgroup (split of K)
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;  // output rows per item = MFMA M
constexpr int kPerSlot = 0, kDedup = 1;
constexpr uint32_t kOOB = 0x80000000u;       // buffer offset beyond every range: load returns 0
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data
constexpr int kSpinLimit = 1 << 17;          // bounded wait on a counter (~0.2 s)

// Workspace sync area at the start of the workspace, the same place for every n
// (so counters never overlap data of another call), one counter per 128-byte
// line (int32 words, kLine words per line):
//   line u,  word 0   h-ready count of unit u: gate/up items of u that wrote h
//   line u,  word 1   down items of unit u that finished reading h
//   line 256 + t      arrivals of units on down row tile t
constexpr int kLine = 32;
constexpr int kMaxDownTiles = 1024;  // d_model <= 16384
constexpr int kSyncWords = kLine * (MOE_MAX_SLOTS + kMaxDownTiles);

// byte offset base + k, or the out-of-range offset when either part is out of range
__device__ __forceinline__ uint32_t cat(uint32_t base, uint32_t k) {
    return ((base | k) & kOOB) ? kOOB : base + k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Data handed between workgroups (h, O) is written and read with the sc1 cache
// policy: agent-coherent accesses, the form of relaxed agent-scope atomics, which
// reach the point of coherence across the XCDs' L2 caches without the cache-wide
// write-back / invalidate of a fence.  A writer waits for its stores to complete
// before the workgroup raises the counter; a reader issues its sc1 loads only
// after it has seen the counter.
constexpr int kSc1 = 16;

__device__ __forceinline__ u32x4 bload_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

// 16-byte load at vector offset vo plus scalar (wave-uniform) offset so.
template <int AUX>
__device__ __forceinline__ u32x4 bload2(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, AUX));
}

__device__ __forceinline__ void stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt = 0: this wave's stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// bf16 16x16x32 MFMA: D += A(16x32) B(32x16).  Lane l supplies A row l%16 and B
// column l%16, elements k = 8*(l/16) .. +8 of the step (any k permutation that A
// and B share gives the same sum).  D: lane l holds rows 4*(l/16)+i, column l%16.
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
    static constexpr int kPer = 16 / kEsize;  // elements per 16-byte lane load
    static constexpr int kStep = 4 * kPer;    // k covered by one wave step
    __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) { return BF16 ? mma_bf16(a, b, c) : mma_f32(a, b, c); }
};

// Offsets of this lane's 16-byte chunk at wave step i (steps s0 .. s0+ns-1 of the
// contraction dimension K) in a row whose byte offset is `base` (kOOB for a row or
// token outside its matrix).  With KF (K a multiple of the step) the lane keeps one
// vector offset per row and the step's k offset is a wave-uniform scalar offset;
// otherwise each step forms a checked vector offset.  Steps past ns read zeros
// through an out-of-range vector offset (scalar offset 0).
template <bool BF16, bool KF>
struct Steps {
    using F = Fmt<BF16>;
    int s0, ns, K, q;
    __device__ uint32_t lane_base(uint32_t base) const {
        return KF ? cat(base, (uint32_t)q * 16u) : base;
    }
    __device__ uint32_t vofs(uint32_t lb, int i) const {
        if (KF) return i < ns ? lb : kOOB;
        const int k = (s0 + i) * F::kStep + q * F::kPer;
        return (i < ns && k < K) ? cat(lb, (uint32_t)k * F::kEsize) : kOOB;
    }
    __device__ uint32_t sofs(int i) const {
        return (KF && i < ns) ? (uint32_t)(s0 + i) * (uint32_t)(F::kStep * F::kEsize) : 0u;
    }
};

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ int atomic_load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Args {
    const char* wg;      // W_gate [N][d_ff][d]
    const char* wu;      // W_up   [N][d_ff][d]
    const char* wd;      // W_down [N][d][d_ff]
    const char* x;       // [n][d]
    const int32_t* ids;  // [n*m]
    const float* w;      // [n*m]
    float* y;            // [n][d]
    char* h;             // bf16: hi [nm][d_ff] then lo [nm][d_ff]; fp32: [nm][d_ff]
    float* O;            // [nm][d]
    int32_t* sync;       // counters, see layout above
    int32_t* info;       // optional [3]
    int32_t n, m, N, d, d_ff;
    int32_t units, T1, T2;
    int32_t accumulate;
};

template <int NB>
struct Smem {
    f32x4 red[kWaves][2][NB][64];  // cross-wave reduction of the MFMA accumulators (NB = row blocks x token tiles)
    int32_t ids[MOE_MAX_SLOTS];
    int32_t grp[MOE_MAX_SLOTS];    // slots of this workgroup's unit, increasing
    uint32_t pres[MOE_MAX_EXPERTS / 32];
    int32_t wsum[kWaves];
    int32_t meta[4];               // e, g, U, flag
};

// Stable grouping of the pass's slots by expert, in LDS, for distinct expert
// number `u` (ids in increasing order).  Also the number U of distinct in-range
// experts and, when want_status, MOE_E_IDS for ids out of range or repeated within
// a token.  Leaves e (or -1), g in sm.meta and the slots in sm.grp.
template <int NB>
__device__ void group_prologue(const Args& a, Smem<NB>& sm, int u, bool want_status) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nm = a.n * a.m;
    const int nwords = (a.N + 31) >> 5;
    if (tid < nwords) sm.pres[tid] = 0u;
    if (tid == 0) sm.meta[3] = 0;
    const int id = tid < nm ? a.ids[tid] : -1;
    const bool valid = tid < nm && id >= 0 && id < a.N;
    if (tid < nm) sm.ids[tid] = valid ? id : -1;
    __syncthreads();
    if (valid) atomicOr(&sm.pres[id >> 5], 1u << (id & 31));
    if (want_status && tid < nm) {
        bool bad = !valid;
        if (valid) {
            const int t = tid / a.m, j = tid - t * a.m;
            for (int jj = 0; jj < j; ++jj) bad |= (sm.ids[t * a.m + jj] == id);
        }
        if (bad) atomicOr(&sm.meta[3], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // prefix popcount over the presence words (<= 32 words)
        const uint32_t word = lane < nwords ? sm.pres[lane] : 0u;
        int c = __popc(word);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        const int U = __shfl(incl, 63, 64);
        const int excl = incl - c;
        if (lane == 0) {
            sm.meta[2] = U;
            sm.meta[0] = -1;
        }
        if (u < U && u >= excl && u < incl) {
            uint32_t wv = word;
            for (int k = u - excl; k > 0; --k) wv &= wv - 1;  // drop the lower set bits
            sm.meta[0] = lane * 32 + __ffs(wv) - 1;
        }
    }
    __syncthreads();
    const int e = sm.meta[0];
    if (e >= 0) {
        const bool f = tid < nm && sm.ids[tid] == e;
        const unsigned long long bal = __ballot(f);
        const int rank = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) sm.wsum[wave] = __popcll(bal);
        __syncthreads();
        int off = 0;
        for (int w = 0; w < wave; ++w) off += sm.wsum[w];
        if (f) sm.grp[off + rank] = tid;
        if (tid == 0) sm.meta[1] = sm.wsum[0] + sm.wsum[1] + sm.wsum[2] + sm.wsum[3];
    } else if (tid == 0) {
        sm.meta[1] = 0;
    }
    __syncthreads();
}

// Bounded wait until *p >= target (one thread).  Returns false on expiry.
__device__ bool wait_count(const int32_t* p, int target) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (atomic_load_agent(p) >= target) return true;
        __builtin_amdgcn_s_sleep(8);
    }
    return false;
}

// ---------------------------------------------------------------------------
// The fused expert operation.
// ---------------------------------------------------------------------------
template <bool BF16, int MODE, int NT, int RB, bool KF>
__global__ __launch_bounds__(kThreads) void k_expert(Args a) {
    using F = Fmt<BF16>;
    // ring depth in steps: operand registers per step are (2*RB + NT) for gate/up
    // and (RB + 2*NT) for down, 4 VGPRs each
    constexpr int P = (2 * RB + NT) <= 3 ? 8 : ((2 * RB + NT) <= 6 ? 4 : 2);
    constexpr int H = P / 2;  // half ring
    constexpr int RT = kTile * RB;  // output rows per item
    __shared__ Smem<NT * RB> sm;
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so step offsets are scalar
    const int lr = lane & 15, q = lane >> 4;
    const int nm = a.n * a.m;
    const int A1 = a.units * a.T1;
    const bool phase1 = (int)blockIdx.x < A1;
    const int item = phase1 ? (int)blockIdx.x : (int)blockIdx.x - A1;
    const int T = phase1 ? a.T1 : a.T2;
    const int u = item / T, t = item - u * T;
    int32_t* hcnt = a.sync + kLine * u;      // this unit's h-ready count
    int32_t* dcnt = hcnt + 1;                // this unit's finished down items
    int32_t* ocnt = a.sync + kLine * (MOE_MAX_SLOTS + t);  // arrivals on this down tile (phase 2)

    // ---- the unit: expert e and its slots sm.grp[0..g) ----
    int e, g;
    const bool want_status = a.info != nullptr && blockIdx.x == 0;
    if (MODE == kDedup || want_status) {
        group_prologue<NT * RB>(a, sm, MODE == kDedup ? u : 0, want_status);
        if (want_status && tid == 0) {
            a.info[0] = sm.meta[2];
            a.info[1] = sm.meta[3] ? MOE_E_IDS : MOE_OK;
            a.info[2] = MOE_OK;  // a bounded wait that expires later overwrites this
        }
    }
    if (MODE == kDedup) {
        e = sm.meta[0];
        g = sm.meta[1];
    } else {
        const int id = a.ids[u];
        e = (id >= 0 && id < a.N) ? id : -1;
        g = e >= 0 ? 1 : 0;
        if (tid == 0) sm.grp[0] = u;
        __syncthreads();
    }

    if (phase1) {
        // ================ gate / up: h for RT rows of d_ff ================
        if (g > 0) {
            const uint32_t mat = (uint32_t)a.d_ff * a.d * F::kEsize;
            const auto rg = rsrc(a.wg + (size_t)e * mat, mat);
            const auto ru = rsrc(a.wu + (size_t)e * mat, mat);
            const auto rx = rsrc(a.x, (uint32_t)(a.n * a.d * F::kEsize));
            const auto rhw = rsrc(a.h, (uint32_t)nm * a.d_ff * 4);  // h region: hi+lo bf16 or fp32
            const int S = (a.d + F::kStep - 1) / F::kStep;
            const int s0 = wave * S / kWaves;
            const Steps<BF16, KF> st{s0, (wave + 1) * S / kWaves - s0, a.d, q};
            const int ns = st.ns;
            uint32_t lrow[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = t * RT + rb * kTile + lr;
                lrow[rb] = st.lane_base(row < a.d_ff ? (uint32_t)row * a.d * F::kEsize : kOOB);
            }
            for (int base = 0; base < g; base += 16 * NT) {
                uint32_t lx[NT];
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int gi = base + tt * 16 + lr;
                    lx[tt] = st.lane_base(gi < g ? (uint32_t)(sm.grp[gi] / a.m) * a.d * F::kEsize : kOOB);
                }
                u32x4 ag[P][RB], au[P][RB], bx[P][NT];
                auto issue = [&](int slot, int j) {  // loads of wave step j into ring slot `slot`
                    const uint32_t so = st.sofs(j);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        ag[slot][rb] = bload2<0>(rg, st.vofs(lrow[rb], j), so);
                        au[slot][rb] = bload2<0>(ru, st.vofs(lrow[rb], j), so);
                    }
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) bx[slot][tt] = bload2<0>(rx, st.vofs(lx[tt], j), so);
                };
#pragma unroll
                for (int i = 0; i < P; ++i) issue(i, i);
                f32x4 accg[RB][NT], accu[RB][NT];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) accg[rb][tt] = accu[rb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                // two halves of the ring: the refill of one half is issued while the
                // other half's data is consumed, so the wave's load stream never drains
                for (int s = 0; s < ns; s += P) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                        for (int i = hh * H; i < hh * H + H; ++i)
#pragma unroll
                            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                                for (int tt = 0; tt < NT; ++tt) {
                                    accg[rb][tt] = F::mma(ag[i][rb], bx[i][tt], accg[rb][tt]);
                                    accu[rb][tt] = F::mma(au[i][rb], bx[i][tt], accu[rb][tt]);
                                }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int i = hh * H; i < hh * H + H; ++i) issue(i, s + i + P);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        sm.red[wave][0][rb * NT + tt][lane] = accg[rb][tt];
                        sm.red[wave][1][rb * NT + tt][lane] = accu[rb][tt];
                    }
                __syncthreads();
                if (wave < RB * NT) {  // wave w finalises row block w / NT, token tile w % NT
                    const int rb = wave / NT, tt = wave - rb * NT;
                    f32x4 G = sm.red[0][0][wave][lane], Uu = sm.red[0][1][wave][lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) {
                        G += sm.red[w][0][wave][lane];
                        Uu += sm.red[w][1][wave][lane];
                    }
                    const int gi = base + tt * 16 + lr;                // output column = lane % 16
                    const int f0 = t * RT + rb * kTile + 4 * q;        // output rows f0 .. f0+3
                    if (gi < g && f0 < a.d_ff) {                       // d_ff % 8 == 0: all 4 rows valid
                        const uint32_t idx = (uint32_t)sm.grp[gi] * a.d_ff + f0;
                        float hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) hv[i] = silu(G[i]) * Uu[i];
                        if (BF16) {
                            uint32_t hi[4], lo[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                hi[i] = bf16_rne(hv[i]);
                                lo[i] = bf16_rne(hv[i] - bf16_to_f32(hi[i]));
                            }
                            const uint32_t half = (uint32_t)nm * a.d_ff * 2;  // bytes of the hi half
                            __builtin_amdgcn_raw_buffer_store_b64(u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)},
                                                                  rhw, idx * 2, 0, kSc1);
                            __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)},
                                                                  rhw, half + idx * 2, 0, kSc1);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(u32x4, f32x4{hv[0], hv[1], hv[2], hv[3]}), rhw, idx * 4, 0, kSc1);
                        }
                    }
                    stores_complete();
                }
                __syncthreads();
            }
        }
        if (tid == 0 && g > 0) atomicAdd(hcnt, 1);  // after the writers' completed stores and the barrier
    } else {
        // ================ down: O for RT rows of d ================
        if (g > 0) {
            const uint32_t mat = (uint32_t)a.d * a.d_ff * F::kEsize;
            const auto rd = rsrc(a.wd + (size_t)e * mat, mat);
            const uint32_t hbytes = (uint32_t)nm * a.d_ff * F::kEsize;
            const auto rh = rsrc(a.h, hbytes);
            const auto rl = rsrc(a.h + (BF16 ? hbytes : 0), hbytes);
            const auto ro = rsrc(a.O, (uint32_t)nm * a.d * 4);
            const int S = (a.d_ff + F::kStep - 1) / F::kStep;
            const int s0 = wave * S / kWaves;
            const Steps<BF16, KF> st{s0, (wave + 1) * S / kWaves - s0, a.d_ff, q};
            const int ns = st.ns;
            uint32_t lrow[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = t * RT + rb * kTile + lr;
                lrow[rb] = st.lane_base(row < a.d ? (uint32_t)row * a.d_ff * F::kEsize : kOOB);
            }
            for (int base = 0; base < g; base += 16 * NT) {
                u32x4 ad[P][RB], bh[P][NT], bl[P][NT];
                uint32_t lh[NT];
                auto issue_a = [&](int slot, int j) {
                    const uint32_t so = st.sofs(j);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) ad[slot][rb] = bload2<0>(rd, st.vofs(lrow[rb], j), so);
                };
                auto issue_b = [&](int slot, int j) {
                    const uint32_t so = st.sofs(j);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        bh[slot][tt] = bload2<kSc1>(rh, st.vofs(lh[tt], j), so);
                        if (BF16) bl[slot][tt] = bload2<kSc1>(rl, st.vofs(lh[tt], j), so);
                    }
                };
#pragma unroll
                for (int i = 0; i < P; ++i) issue_a(i, i);  // weights first
                if (base == 0) {
                    if (tid == 0 && !wait_count(hcnt, a.T1) && a.info) a.info[2] = MOE_E_HIP;
                    __syncthreads();  // h loads (sc1) below are issued after the count was seen
                }
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int gi = base + tt * 16 + lr;
                    lh[tt] = st.lane_base(gi < g ? (uint32_t)sm.grp[gi] * a.d_ff * F::kEsize : kOOB);
                }
#pragma unroll
                for (int i = 0; i < P; ++i) issue_b(i, i);
                f32x4 acc[RB][NT];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) acc[rb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s < ns; s += P) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                        for (int i = hh * H; i < hh * H + H; ++i)
#pragma unroll
                            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                                for (int tt = 0; tt < NT; ++tt) {
                                    acc[rb][tt] = F::mma(ad[i][rb], bh[i][tt], acc[rb][tt]);
                                    if (BF16) acc[rb][tt] = F::mma(ad[i][rb], bl[i][tt], acc[rb][tt]);
                                }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int i = hh * H; i < hh * H + H; ++i) {
                            issue_a(i, s + i + P);
                            issue_b(i, s + i + P);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) sm.red[wave][0][rb * NT + tt][lane] = acc[rb][tt];
                __syncthreads();
                if (wave < RB * NT) {
                    const int rb = wave / NT, tt = wave - rb * NT;
                    f32x4 v = sm.red[0][0][wave][lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) v += sm.red[w][0][wave][lane];
                    const int gi = base + tt * 16 + lr;
                    const int i0 = t * RT + rb * kTile + 4 * q;
                    if (gi < g && i0 < a.d)  // d % 8 == 0: rows i0..i0+3 all valid
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                                               ((uint32_t)sm.grp[gi] * a.d + i0) * 4, 0, kSc1);
                    stores_complete();
                }
                __syncthreads();
            }
            // the unit's last down item resets the unit's counters for the next call
            // (every down item of the unit has seen the full h-ready count by now)
            if (tid == 0 && atomicAdd(dcnt, 1) == a.T2 - 1) {
                __hip_atomic_store(hcnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dcnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // arrival on this row tile; the last unit to arrive combines its rows
        if (tid == 0) {
            const int old = atomicAdd(ocnt, 1);  // after the writers' completed stores and the barrier
            s_last = old == a.units - 1;
            if (s_last) __hip_atomic_store(ocnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // all arrived
        }
        __syncthreads();  // O loads (sc1) below are issued after the last arrival was seen
        if (s_last) {
            const int i0 = t * RT;
            const int rows = min(RT, a.d - i0);
            for (int o = tid; o < a.n * rows; o += kThreads) {
                const int tok = o / rows, i = i0 + (o - tok * rows);
                float acc = 0.f;
                for (int j = 0; j < a.m; ++j) {
                    const int s = tok * a.m + j;
                    const int id = a.ids[s];
                    if (id >= 0 && id < a.N)
                        acc = fmaf(a.w[s], __hip_atomic_load(a.O + (size_t)s * a.d + i, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT), acc);
                }
                float* yp = a.y + (size_t)tok * a.d + i;
                *yp = a.accumulate ? *yp + acc : acc;
            }
        }
    }
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
    for (int dd = 1; dd < 256; dd <<= 1) {
        int a0 = 0, a1 = 0;
        if (tid >= dd) {
            a0 = s_part[tid - dd][0];
            a1 = s_part[tid - dd][1];
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
    const int64_t es = d->dtype == MOE_BF16 ? 2 : 4;
    // one expert matrix must be addressable by a 31-bit buffer offset
    if ((int64_t)d->d_model * d->d_ff * es > (1ll << 31) - 4096) return MOE_E_INVAL;
    if ((d->d_model + kTile - 1) / kTile > kMaxDownTiles) return MOE_E_INVAL;  // d_model <= 16384
    return MOE_OK;
}

struct Plan {
    int units, T1, T2, nt, rb;
    size_t h_off, o_off, sync_off, total;
};

Plan plan_for(const moe_layer_desc* d, int32_t n, int kind) {
    Plan p;
    const int nm = n * d->m;
    p.units = kind == MOE_KIND_SLOT ? nm : (nm < d->N ? nm : d->N);
    p.nt = kind == MOE_KIND_SLOT ? 1 : (n <= 16 ? 1 : (n <= 32 ? 2 : 4));
    p.rb = p.nt == 4 ? 1 : 2;  // rows per item = 16 * rb; row blocks x token tiles <= 4
    p.T1 = (d->d_ff + kTile * p.rb - 1) / (kTile * p.rb);
    p.T2 = (d->d_model + kTile * p.rb - 1) / (kTile * p.rb);
    p.sync_off = 0;
    p.h_off = (size_t)kSyncWords * 4;
    p.o_off = p.h_off + align_up((size_t)nm * d->d_ff * 4);
    p.total = p.o_off + align_up((size_t)nm * d->d_model * 4);
    return p;
}

template <bool BF16, int MODE, int NT, int RB>
void launch(const Args& args, int grid, hipStream_t st) {
    constexpr int step = Fmt<BF16>::kStep;
    if (args.d % step == 0 && args.d_ff % step == 0)
        hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true>), dim3(grid), dim3(kThreads), 0, st, args);
    else
        hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, false>), dim3(grid), dim3(kThreads), 0, st, args);
}

template <int MODE>
int run_expert(const moe_layer_desc* d, const moe_layer_weights* W, const void* x, const int32_t* ids,
               const float* w, int32_t n, float* y, int32_t* info, void* ws, size_t ws_bytes, void* stream,
               void* const* events, int32_t n_events) {
    int rc = check_desc(d, n);
    if (rc != MOE_OK) return rc;
    if (!W || !W->w_gate || !W->w_up || !W->w_down || !x || !ids || !w || !y || !ws) return MOE_E_INVAL;
    if (!aligned16(W->w_gate) || !aligned16(W->w_up) || !aligned16(W->w_down) || !aligned16(x) || !aligned16(y))
        return MOE_E_INVAL;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_E_INVAL;
    const int kind = MODE == kPerSlot ? MOE_KIND_SLOT : MOE_KIND_DEDUP;
    const Plan p = plan_for(d, n, kind);
    if (ws_bytes < p.total) return MOE_E_WORKSPACE;
    if (events) {
        if (n_events != 2 || !events[0] || !events[1]) return MOE_E_INVAL;
    } else if (n_events != 0) {
        return MOE_E_INVAL;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* wsb = reinterpret_cast<char*>(ws);
    Args args;
    args.wg = reinterpret_cast<const char*>(W->w_gate);
    args.wu = reinterpret_cast<const char*>(W->w_up);
    args.wd = reinterpret_cast<const char*>(W->w_down);
    args.x = reinterpret_cast<const char*>(x);
    args.ids = ids;
    args.w = w;
    args.y = y;
    args.h = wsb + p.h_off;
    args.O = reinterpret_cast<float*>(wsb + p.o_off);
    args.sync = reinterpret_cast<int32_t*>(wsb + p.sync_off);
    args.info = info;
    args.n = n;
    args.m = d->m;
    args.N = d->N;
    args.d = d->d_model;
    args.d_ff = d->d_ff;
    args.units = p.units;
    args.T1 = p.T1;
    args.T2 = p.T2;
    args.accumulate = (d->flags & MOE_FLAG_ACCUMULATE) ? 1 : 0;
    const int grid = p.units * (p.T1 + p.T2);
    (void)hipGetLastError();
    if (events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[0]), st);
    const bool bf = d->dtype == MOE_BF16;
    if (bf) {
        if (p.nt == 1) launch<true, MODE, 1, 2>(args, grid, st);
        else if (p.nt == 2) launch<true, MODE, 2, 2>(args, grid, st);
        else launch<true, MODE, 4, 1>(args, grid, st);
    } else {
        if (p.nt == 1) launch<false, MODE, 1, 2>(args, grid, st);
        else if (p.nt == 2) launch<false, MODE, 2, 2>(args, grid, st);
        else launch<false, MODE, 4, 1>(args, grid, st);
    }
    if (events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[1]), st);
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
    return plan_for(desc, n, kind).total;
}

int moe_kernels_per_call(int32_t kind) {
    if (kind != MOE_KIND_SLOT && kind != MOE_KIND_DEDUP) return MOE_E_INVAL;
    return 1;
}

int moe_expert_perslot(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                       const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info, void* ws,
                       size_t ws_bytes, void* hip_stream) {
    return run_expert<kPerSlot>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, nullptr, 0);
}

int moe_expert_dedup(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                     const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info, void* ws,
                     size_t ws_bytes, void* hip_stream) {
    return run_expert<kDedup>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, nullptr, 0);
}

int moe_expert_perslot_ev(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                          const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info, void* ws,
                          size_t ws_bytes, void* hip_stream, void* const* events, int32_t n_events) {
    if (!events) return MOE_E_INVAL;
    return run_expert<kPerSlot>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, events, n_events);
}

int moe_expert_dedup_ev(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                        const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info, void* ws,
                        size_t ws_bytes, void* hip_stream, void* const* events, int32_t n_events) {
    if (!events) return MOE_E_INVAL;
    return run_expert<kDedup>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, events, n_events);
}

}  // extern "C"
