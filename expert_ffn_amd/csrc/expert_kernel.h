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
//     contraction dimension K into four contiguous ranges, or, with tiled weights
//     (blocks of 16 rows x one K step, see TSteps), take every fourth step so that
//     at each step they read adjacent blocks.
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
//
// Internal to the library: this header holds the kernel, its helpers and its
// launch templates; expert_launch.hip instantiates them once per (dtype, kernel,
// shared experts), so the variants compile in parallel, and moe_expert.hip plans
// and dispatches the launches.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "moe_expert.h"

namespace moe_k {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kWaves = 4;  // waves per workgroup (split of K)
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;  // output rows per item = MFMA M
constexpr int kPerSlot = 0, kDedup = 1;
constexpr int kLayPlain = 0, kLayPacked = 1, kLayTiled = 2;  // weight layouts (MOE_FLAG_*)
constexpr uint32_t kOOB = 0x80000000u;       // buffer offset beyond every range: load returns 0
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data
constexpr int kSpinLimit = 1 << 17;          // bounded wait on a counter (~0.2 s)

// Workspace sync area at the start of the workspace, the same place for every n
// (so counters never overlap data of another call), one counter per 128-byte
// line (int32 words, kLine words per line):
//   line u,  word 0   h-ready count of unit u: gate/up items of u that wrote h
//   line u,  word 1   down items of unit u that finished reading h
//   line 256 + t      arrivals of units on down row tile t
//   line 1280 + c     contributions to split gate/up tile c
constexpr int kLine = 32;
constexpr int kMaxDownTiles = 1024;  // d_model <= 16384
constexpr int kCUs = 256;            // compute units: the gate/up split balances work over them
constexpr int kMaxSplitTiles = 2 * kCUs;
constexpr int kMaxContrib = 3;       // work groups sharing one split gate/up tile
constexpr int kSyncWords = kLine * (MOE_MAX_SLOTS + kMaxDownTiles + kMaxSplitTiles);

// byte offset base + k, or the out-of-range offset when either part is out of range
__device__ __forceinline__ uint32_t cat(uint32_t base, uint32_t k) {
    return ((base | k) & kOOB) ? kOOB : base + k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

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
// A wave's steps are s0, s0 + SS, s0 + 2 SS, ...: a contiguous range (SS = 1) or,
// with tiled weights, every kWaves-th step (SS = kWaves).
template <bool BF16, bool KF, int SS = 1>
struct Steps {
    using F = Fmt<BF16>;
    int s0, ns, K, q;
    __device__ uint32_t lane_base(uint32_t base) const {
        return KF ? cat(base, (uint32_t)q * 16u) : base;
    }
    __device__ int step(int i) const { return s0 + SS * i; }
    __device__ uint32_t vofs(uint32_t lb, int i) const {
        if (KF) return i < ns ? lb : kOOB;
        const int k = step(i) * F::kStep + q * F::kPer;
        return (i < ns && k < K) ? cat(lb, (uint32_t)k * F::kEsize) : kOOB;
    }
    __device__ uint32_t sofs(int i) const {
        return (KF && i < ns) ? (uint32_t)step(i) * (uint32_t)(F::kStep * F::kEsize) : 0u;
    }
};

// Tiled weights: a matrix of R rows and K contraction columns (R a multiple of 16,
// K of the step) in blocks of 16 rows x one step (64 bytes a row, 1 KB a block);
// block (r16, s) at byte (r16 * S + s) * 1 KB with S = K / step, and in a block lane
// l's 16 bytes, row l % 16 and k-group l / 16, at byte 16 l.  One load instruction
// reads one whole block.  With the wave-interleaved step order (wave w takes steps
// w, w + 4, ...) the four waves of a work group read adjacent blocks at each step.
constexpr uint32_t kBlock = 1024;
struct TSteps {
    int s0, ns;  // steps s0, s0 + kWaves, ...
    __device__ static uint32_t lane_base(bool ok, int r16, int S, int lane) {
        return ok ? (uint32_t)r16 * (uint32_t)S * kBlock + (uint32_t)lane * 16u : kOOB;
    }
    __device__ uint32_t vofs(uint32_t lb, int i) const { return i < ns ? lb : kOOB; }
    __device__ uint32_t sofs(int i) const { return i < ns ? (uint32_t)(s0 + kWaves * i) * kBlock : 0u; }
};

// steps of [k0, k0 + len) that wave w takes in the interleaved order
__device__ __forceinline__ int interleaved_steps(int len, int w) {
    return len > w ? (len - w + kWaves - 1) / kWaves : 0;
}

// W_down packed in blocks of 8 columns, [N][d_ff/8][d_model][8] (element (i, f) at
// byte ((f/8)*d + i)*8*E + (f%8)*E): the 8*k-th .. 8*k+7-th hidden columns of all
// output rows are contiguous.  Offsets of this lane's 16-byte chunk of row i at wave
// step i of the d_ff contraction.  With KF the step offset is a scalar offset
// (d_ff a multiple of the step: it never passes the matrix); otherwise the chunk
// is formed in the vector offset and checked against d_ff.
template <bool BF16, bool KF>
struct PSteps {
    using F = Fmt<BF16>;
    int s0, ns, K, d, q;
    __device__ uint32_t lane_base(bool ok, int row) const {
        if (!ok) return kOOB;
        const uint32_t f = (uint32_t)q * F::kPer;  // this lane's columns within a step
        return ((f / 8) * (uint32_t)d + (uint32_t)row) * 8u * F::kEsize + (f % 8) * F::kEsize;
    }
    __device__ uint32_t vofs(uint32_t lb, int i) const {
        if (KF) return i < ns ? lb : kOOB;
        const int k = (s0 + i) * F::kStep + q * F::kPer;
        return (i < ns && k < K) ? cat(lb, (uint32_t)(s0 + i) * 64u * (uint32_t)d) : kOOB;
    }
    __device__ uint32_t sofs(int i) const {
        return (KF && i < ns) ? (uint32_t)(s0 + i) * 64u * (uint32_t)d : 0u;
    }
};

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// a value that is the same in every lane, kept in a scalar register
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int atomic_load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Args {
    const char* wg;      // W_gate [N][d_ff][d] (or tiled)
    const char* wu;      // W_up   [N][d_ff][d] (or tiled)
    const char* wd;      // W_down [N][d][d_ff] (or packed, or tiled)
    const char* wgs;     // always-on (shared) experts: W_gate [n_shared][d_ff][d], or null
    const char* wus;     // W_up [n_shared][d_ff][d]
    const char* wds;     // W_down [n_shared][d][d_ff], layout as wd
    const char* x;       // [n][d]
    const int32_t* ids;  // [n*m]
    const float* w;      // [n*m]
    float* y;            // [n][d]
    char* h;             // bf16: hi [nslot][d_ff] then lo [nslot][d_ff]; fp32: [nslot][d_ff]
    float* O;            // [nslot][ks][d]: per slot and contraction part
    int32_t* sync;       // counters, see layout above
    int32_t* info;       // optional [3]
    int32_t n, m, N, d, d_ff;
    int32_t units, T1, T2;
    int32_t units_r;     // routed units; units units_r .. units-1 are the shared experts
    int32_t ks;          // down items per (unit, row tile): parts of the d_ff contraction
    int32_t n_shared;
    int32_t nslot;       // rows of h and O: routed slots t*m + j, then shared slots nm + s*n + t
    int32_t accumulate;
    int32_t gl;          // down items in register mode: tokens of h staged in LDS at a time
    int32_t g1;          // gate/up work groups (they take the first g1 block ids)
    int32_t S1;          // K steps of one gate/up row tile
    int32_t split_ok;    // the workspace holds the partial sums of split gate/up tiles
    int32_t reg_wgs;     // deduplicating kernel: most work groups (gate/up and down) for register-mode down items
    float* part;         // split gate/up tiles: partial sums [kMaxContrib][nslot][d_ff][gate, up]
};

// token of a slot: routed slot t*m + j, shared slot n*m + s*n + t
__device__ __forceinline__ int slot_tok(const Args& a, int slot) {
    const int nm = a.n * a.m;
    return slot < nm ? slot / a.m : (slot - nm) % a.n;
}

// LDS bytes for the h a register-mode down item stages (gl tokens of a chunk).
// Variants whose cross-wave reduction array holds at least that much (two or more
// token tiles: 32 KB) stage h in that array itself, which no other part of a down
// item uses while h is read, and need no dynamic LDS: a dedup pass of the 32-node
// tree then keeps 3 work groups per compute unit (its registers' limit) instead of 2.
constexpr int kHsBudget = 32 * 1024;
__host__ __device__ constexpr bool hs_in_red(int nb) { return 16 * kWaves * 2 * nb * 64 >= kHsBudget; }

template <int NB>
struct Smem {
    f32x4 red[kWaves][2][NB][64];  // cross-wave reduction of the MFMA accumulators (NB = row blocks x token tiles)
    int32_t ids[MOE_MAX_SLOTS];
    int32_t grp[MOE_MAX_SLOTS];    // slots of this workgroup's unit, increasing
    uint32_t pres[MOE_MAX_EXPERTS / 32];
    int32_t id_status;             // set for ids out of range or repeated within a token
    float cw[MOE_MAX_SLOTS];       // down items: routing weight of each slot, for the combine
    int32_t cok[MOE_MAX_SLOTS];    // down items: the slot's id is in range
};

// The pass's ids in LDS (ids out of range as -1) and the presence bitmap of the
// experts they name; with want_status, sm.id_status is set for ids out of range or
// repeated within a token (read after the call by thread 0).  Loaded once per work
// group, at the kernel's start (no earlier use of sm): the unit selections below read
// it.  Ends with a barrier.
template <int NB>
__device__ void load_ids(const Args& a, Smem<NB>& sm, bool want_status) {
    const int tid = threadIdx.x;
    const int nm = a.n * a.m;
    // the id load first, so that the kernel-argument loads it depends on go out
    // together at the kernel's start
    const int id = tid < nm ? a.ids[tid] : -1;
    const int nwords = (a.N + 31) >> 5;
    if (tid < nwords) sm.pres[tid] = 0u;
    if (tid == 0) sm.id_status = 0;
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
        if (bad) atomicOr(&sm.id_status, 1);
    }
    __syncthreads();
}

// Stable grouping of the pass's slots by expert, from what load_ids left in LDS: the
// number U of distinct experts and, for distinct expert number `u` (ids in increasing
// order; u < 0 or u >= U: none), its id e (else -1) and, with `group`, its slots,
// increasing, in sm.grp[0..g).  One LDS round trip (the presence words and, with
// `group`, the ids, read together); the walk over the presence words runs on the
// scalar unit (readlane) and the group is formed with ballots, so the chain of
// dependent LDS operations a shuffle scan would make stays off the path to the
// first weight load.  Every wave computes the same result itself (and writes all of
// sm.grp), so no barrier is needed after it; the barrier before it keeps the
// previous unit's reads of sm.grp ahead of the writes.
template <int NB>
__device__ void select_unit(const Args& a, Smem<NB>& sm, int u, bool group, int& e_out, int& g_out, int& U_out,
                            bool barrier = true) {
    constexpr int kChunks = MOE_MAX_SLOTS / 64;
    const int lane = threadIdx.x & 63;
    const int nm = a.n * a.m;
    const int nwords = (a.N + 31) >> 5;  // <= 32
    if (barrier) __syncthreads();
    const uint32_t word = lane < nwords ? sm.pres[lane] : 0u;
    int idv[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) idv[i] = (group && lane + 64 * i < nm) ? sm.ids[lane + 64 * i] : -1;
    // distinct expert u: the (u - U)-th set bit of the word where the running count U
    // passes u (words in increasing order, bits in increasing order)
    int U = 0, e = -1;
    for (int w = 0; w < nwords; ++w) {
        uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)word, w);
        const int c = __popc(wv);
        if (u >= U && u < U + c) {
            for (int k = u - U; k > 0; --k) wv &= wv - 1u;  // drop the lower set bits
            e = w * 32 + __ffs(wv) - 1;
        }
        U += c;
    }
    int g = 0;
    if (group && e >= 0) {
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            if (64 * i < nm) {
                const bool f = idv[i] == e;
                const unsigned long long bal = __ballot(f);
                if (f) sm.grp[g + __popcll(bal & below)] = lane + 64 * i;
                g += __popcll(bal);
            }
        }
    }
    e_out = e;
    g_out = g;
    U_out = U;
}

// Gate/up work groups for `tiles` row tiles of S1 K steps: the (unit, tile, K step)
// space is cut into kCUs equal shares when there are between half the compute units
// and `upper` tiles, each tile into two shares when there are fewer than half (and K
// has two steps), else one work group per tile; `split_ok` false forbids cutting (no
// room for partial sums).  Non-decreasing in `tiles` (upper >= kCUs).
// upper: 2 kCUs for the per-slot kernel, kDedupSplitUpper for the deduplicating one.
// Same box, Qwen3-shaped layer x48 (zipf) and DeepSeek-V2-Lite-shaped layer, 8 windows
// per n, two rounds agreeing within 0.1 us: the deduplicating kernel cutting below
// 320 tiles against 288 is 0.3 us per layer faster at n = 2 (Qwen3, 12-13 distinct
// experts: 288 or 312 tiles) and the same elsewhere; below 512 it is 1-2.7 us slower
// at n = 3..8; the per-slot kernel's 384-tile pass (Qwen3 shape, n = 2) is 3.2 us
// faster cut (29.8 against 33.0 us).  A work group's own stream is bounded by the
// loads it keeps in flight, so one work group per tile keeps more bytes in flight;
// below ~300 tiles the compute units with two tiles finish last by a whole tile, and
// the cut wins.
constexpr int kDedupSplitUpper = 320;
__host__ __device__ inline int gate_up_groups(int tiles, int S1, bool split_ok, int upper) {
    const bool few = tiles * 2 < kCUs && S1 >= 2;
    const bool split = ((tiles * 2 >= kCUs && tiles < upper) || few) && split_ok;
    return !split ? tiles : (few ? 2 * tiles : kCUs);
}

// Remainder cut, for large tiles (kCutMinS1 K steps or more, where one more whole
// tile on a compute unit costs tens of microseconds) in passes of `upper` tiles or
// more: the whole rounds of kCUs tiles one work group each, then the remaining
// tiles' K steps cut into min(kCUs, 2 rem) equal contiguous shares, each at least
// half a tile, so that a tile meets at most kMaxContrib shares.  Below `upper` the
// rule of gate_up_groups.  Only the kernels built with RC apply it (a separate
// variant: the others' code is unchanged).
constexpr int kCutMinS1 = 128;
__host__ __device__ inline int rc_whole(int tiles) { return kCUs * (tiles / kCUs); }
__host__ __device__ inline int gate_up_groups_rc(int tiles, int S1, bool split_ok, int upper) {
    if (!split_ok || tiles < upper || S1 < 2) return gate_up_groups(tiles, S1, split_ok, upper);
    const int rem = tiles - rc_whole(tiles);
    return rem == 0 ? tiles : rc_whole(tiles) + (2 * rem < kCUs ? 2 * rem : kCUs);
}
// A pass planned by gate_up_groups_rc with a remainder (g1 != tiles, tiles >= upper):
// work group wi's share [lbeg, lend) of the (tile, K step) space, and a tile's
// contributors first .. last (whole tiles: the one work group; a remainder tile:
// the shares that meet it, in K order, the finaliser last).  A cut tile's counter
// is its index among the remainder tiles, tile - W < kCUs.
struct RcPlan {
    int S1, W, G2, Lr;  // whole-tile work groups, remainder shares, remainder K steps
    __host__ __device__ RcPlan(int tiles, int s1, int g1)
        : S1(s1), W(rc_whole(tiles)), G2(g1 - rc_whole(tiles)), Lr((tiles - rc_whole(tiles)) * s1) {}
    __host__ __device__ int lbeg(int wi) const { return wi < W ? wi * S1 : W * S1 + (wi - W) * Lr / G2; }
    __host__ __device__ int lend(int wi) const { return wi < W ? (wi + 1) * S1 : W * S1 + (wi - W + 1) * Lr / G2; }
    __host__ __device__ int first(int tile) const {
        return tile < W ? tile : W + (((tile - W) * S1 + 1) * G2 - 1) / Lr;
    }
    __host__ __device__ int last(int tile) const {
        return tile < W ? tile : W + (((tile - W) * S1 + S1) * G2 - 1) / Lr;
    }
};

// Down items of a pass of `units` units whose gate/up work takes g1 work groups: in
// register mode (rbr row blocks an item, the whole d_ff contraction) when it is
// allowed and either its items hold 32 or 64 rows (rbr >= 2, at least a streaming
// item's rows) or the pass's work groups, the g1 and these items, number at most reg_wgs
// (about 11/4 rounds of what the compute units hold at once); else streaming (rbs
// row blocks an item), the d_ff contraction of each (unit, row tile) cut into ks_s
// parts.  Register-mode items of 16 rows measured slower than streaming items of
// 32 from 3 rounds on; those of 32 rows were faster at every round count measured
// (Qwen3 shape per-slot, 3.4 to 5.5 rounds at n = 5..8: 5-6 % per pass).
constexpr int kMaxKs = 4;  // contraction parts of a streaming down item, at most
struct DownShape {
    int reg, T2, ks;
};
__host__ __device__ inline DownShape down_shape(int units, int g1, int d, bool reg_allowed, int rbr, int rbs,
                                                int reg_wgs, int ks_s) {
    const int t2r = (d + kTile * rbr - 1) / (kTile * rbr);
    if (reg_allowed && (rbr >= 2 || g1 + units * t2r <= reg_wgs)) return DownShape{1, t2r, 1};
    return DownShape{0, (d + kTile * rbs - 1) / (kTile * rbs), ks_s};
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
// Gate/up products of one segment of a row tile: rows t*RT .. t*RT+RT-1 of d_ff
// for the unit (expert e, slots sm.grp[0..g)), over K steps k0 .. k1-1 of the
// contraction, split over the four waves.  A segment that covers all of K
// (nc == 1) finalises h = silu(gate) * up at once.  Otherwise the tile is shared
// by nc consecutive work groups, contributor j = 0 .. nc-1 in K order: the first
// nc-1 store their partial sums and count in; the last (the finaliser, highest
// work-group id, so every work group it waits for was dispatched before it and
// never waits on a higher id) waits for the count, adds the partials in
// contributor order and then its own, and finalises h.  Returns true in the work
// group that finalised the tile.
// ---------------------------------------------------------------------------
template <bool BF16, int NT, int RB, bool KF, int P, bool SH, bool TL>
__device__ __forceinline__ bool gate_up(const Args& a, Smem<NT * RB>& sm, int e, bool sh, int g, int t, int k0,
                                        int k1, int tile, int nc, int j) {
    using F = Fmt<BF16>;
    constexpr int H = P / 2;        // half ring
    constexpr int RT = kTile * RB;  // output rows of a tile
    // lane-dependent values are formed afresh for every segment (an opaque copy of
    // the thread id), not hoisted out of the caller's loop over segments, where they
    // would hold registers through the load ring
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int nslot = SH ? a.nslot : a.n * a.m;
    const uint32_t mat = (uint32_t)a.d_ff * a.d * F::kEsize;
    const auto rg = rsrc((SH && sh ? a.wgs : a.wg) + (size_t)e * mat, mat);
    const auto ru = rsrc((SH && sh ? a.wus : a.wu) + (size_t)e * mat, mat);
    const auto rx = rsrc(a.x, (uint32_t)(a.n * a.d * F::kEsize));
    int32_t* tc = a.sync + kLine * (MOE_MAX_SLOTS + kMaxDownTiles + tile);  // split tile: partials stored
    const int len = k1 - k0;
    // tiled weights: wave w takes steps k0 + w, k0 + w + 4, ...; else a contiguous quarter
    const int s0 = TL ? k0 + wave : k0 + wave * len / kWaves;
    const Steps<BF16, KF, TL ? kWaves : 1> st{s0, TL ? interleaved_steps(len, wave) : k0 + (wave + 1) * len / kWaves - s0,
                                             a.d, q};
    const TSteps tst{s0, st.ns};
    const int ns = st.ns;
    // h = silu(G) * U for rows f0 .. f0+3 of slot `slot` (bf16: hi and lo halves)
    auto store_h = [&](f32x4 G, f32x4 Uu, int slot, int f0) {
        const auto rhw = rsrc(a.h, (uint32_t)nslot * a.d_ff * 4);  // h region: hi+lo bf16 or fp32
        const uint32_t idx = (uint32_t)slot * a.d_ff + f0;
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
            const uint32_t half = (uint32_t)nslot * a.d_ff * 2;  // bytes of the hi half
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)}, rhw, idx * 2,
                                                  0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)}, rhw,
                                                  half + idx * 2, 0, kSc1);
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{hv[0], hv[1], hv[2], hv[3]}), rhw,
                                                   idx * 4, 0, kSc1);
        }
    };
    uint32_t lrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = t * RT + rb * kTile + lr;
        const int r16 = t * RB + rb;  // tiled: row block (d_ff a multiple of 16)
        lrow[rb] = TL ? TSteps::lane_base(r16 * kTile < a.d_ff, r16, a.S1, lane)
                      : st.lane_base(row < a.d_ff ? (uint32_t)row * a.d * F::kEsize : kOOB);
    }
    for (int base = 0; base < g; base += 16 * NT) {
        uint32_t lx[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int gi = base + tt * 16 + lr;
            const int tok = gi < g ? (SH ? slot_tok(a, sm.grp[gi]) : sm.grp[gi] / a.m) : 0;
            lx[tt] = st.lane_base(gi < g ? (uint32_t)tok * a.d * F::kEsize : kOOB);
        }
        u32x4 ag[P][RB], au[P][RB], bx[P][NT];
        auto issue = [&](int slot, int j) {  // loads of wave step j into ring slot `slot`
            const uint32_t so = st.sofs(j);
            const uint32_t wo = TL ? tst.sofs(j) : so;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint32_t vo = TL ? tst.vofs(lrow[rb], j) : st.vofs(lrow[rb], j);
                ag[slot][rb] = bload2<0>(rg, vo, wo);
                au[slot][rb] = bload2<0>(ru, vo, wo);
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) bx[slot][tt] = bload2<0>(rx, st.vofs(lx[tt], j), so);
        };
        // the ring's first loads in slot order (a scheduling barrier after each slot):
        // the loop's waits then count only the other half's loads as outstanding,
        // instead of waiting for every load whenever the prologue order differs
#pragma unroll
        for (int i = 0; i < P; ++i) {
            issue(i, i);
            __builtin_amdgcn_sched_barrier(0);
        }
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
        // the finaliser of a split tile waits (bounded) until the other nc-1
        // contributors, all of lower work-group id, have stored their partials
        if (base == 0 && nc > 1 && j == nc - 1 && tid == 0 && !wait_count(tc, nc - 1) && a.info)
            a.info[2] = MOE_E_HIP;
        __syncthreads();  // partial loads (sc1) below are issued after the count was seen
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
                const int slot = sm.grp[gi];
                if (nc == 1) {
                    store_h(G, Uu, slot, f0);
                } else {
                    // partial of contributor jj at jj*pstride + pb: (gate, up) pairs of rows f0 .. f0+3
                    const auto rp = rsrc(a.part, (uint32_t)kMaxContrib * nslot * a.d_ff * 8);
                    const uint32_t pstride = (uint32_t)nslot * a.d_ff * 8;
                    const uint32_t pb = ((uint32_t)slot * a.d_ff + f0) * 8;
                    if (j < nc - 1) {
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{__float_as_uint(G[0]), __float_as_uint(Uu[0]), __float_as_uint(G[1]),
                                  __float_as_uint(Uu[1])},
                            rp, j * pstride + pb, 0, kSc1);
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{__float_as_uint(G[2]), __float_as_uint(Uu[2]), __float_as_uint(G[3]),
                                  __float_as_uint(Uu[3])},
                            rp, j * pstride + pb + 16, 0, kSc1);
                    } else {
                        // the others' partials, all loads in flight, added in contributor
                        // order, then this work group's own
                        u32x4 pv[kMaxContrib - 1][2];
#pragma unroll
                        for (int jj = 0; jj < kMaxContrib - 1; ++jj) {
                            pv[jj][0] = bload_sc1(rp, jj < j ? jj * pstride + pb : kOOB);
                            pv[jj][1] = bload_sc1(rp, jj < j ? jj * pstride + pb + 16 : kOOB);
                        }
                        f32x4 Gs = f32x4{0.f, 0.f, 0.f, 0.f}, Us = Gs;
#pragma unroll
                        for (int jj = 0; jj < kMaxContrib - 1; ++jj) {
                            if (jj < j) {
                                Gs += f32x4{__uint_as_float(pv[jj][0].x), __uint_as_float(pv[jj][0].z),
                                            __uint_as_float(pv[jj][1].x), __uint_as_float(pv[jj][1].z)};
                                Us += f32x4{__uint_as_float(pv[jj][0].y), __uint_as_float(pv[jj][0].w),
                                            __uint_as_float(pv[jj][1].y), __uint_as_float(pv[jj][1].w)};
                            }
                        }
                        store_h(Gs + G, Us + Uu, slot, f0);
                    }
                }
            }
            stores_complete();
        }
        __syncthreads();
    }
    if (nc == 1) return true;
    if (j < nc - 1) {
        if (tid == 0) atomicAdd(tc, 1);  // after the writers' completed stores and the barrier
        return false;
    }
    if (tid == 0) __hip_atomic_store(tc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // all nc-1 were counted
    return true;
}

// ---------------------------------------------------------------------------
// The fused expert operation.
// ---------------------------------------------------------------------------
// Down items hold all of their W_down rows in registers (register mode, DPF > 0)
// when a wave's share of the contraction is at most kPF steps: 16 rows (DPF = 1), or,
// when it is at most kPF / 2 steps, 32 rows in the same registers (DPF = 2: half as
// many down items, so more of them are resident while gate/up runs), or 64 rows in
// twice the registers (DPF = 4, one token tile: 153-159 VGPRs and AGPRs, 3 waves per
// SIMD); the deduplicating kernel with one token tile also holds 32 rows of up to
// kPF steps (DPF = 3, the same registers as DPF = 4): DeepSeek-V2-Lite shape dedup
// 0.8-3.3 us faster at n = 1..4, the per-slot kernel not faster so.  Same box, Qwen3 shape x48: 64-row items made the deduplicating kernel
// 0.4-2.4 us per layer faster at every n (n = 8: 47.6 -> 45.2 us) and the per-slot
// kernel, giving up its cap of 4 waves per SIMD for them, 0.2-3.5 us (n = 1 23.6 ->
// 23.0 us, n = 8 75.9 -> 72.4 us): fewer items pay the fixed latencies of the
// hand-off.
constexpr int kPF = 12;
constexpr int kSL = 4;  // register mode: h staging loads in flight per thread

// ---------------------------------------------------------------------------
// One down work group: item `item` of the pass's units * T2 * ks down items, O for
// RT2 rows of d of one unit (or one contraction part of them), then its arrival on
// the row tile and, for the last unit to arrive, the combine.  DPF > 0: register
// mode (RBR row blocks, W_down in registers); DPF == 0: streaming (RB row blocks).
// Its own function so that each form is compiled on its own: the deduplicating
// kernel, which picks the form on the device, calls both (one call runs).
// ---------------------------------------------------------------------------
template <bool BF16, int MODE, int NT, int RB, bool KF, int DPF, int LAY, bool SH, typename Resolve>
__device__ __forceinline__ void down_work(const Args& a, Smem<NT * RB>& sm, int& s_last, int item, int units, int T2,
                                          int ks, Resolve&& resolve) {
    using F = Fmt<BF16>;
    constexpr bool PK = LAY == kLayPacked, TL = LAY == kLayTiled;
    constexpr int P = (2 * RB + NT) <= 3 ? 8 : ((2 * RB + NT) <= 6 ? 4 : 2);  // ring depth, as in the kernel
    constexpr int H = P / 2;
    constexpr int RBR = DPF == 4 ? 4 : (DPF == 2 || DPF == 3 ? 2 : 1), RBS = RB;  // row blocks: register mode, streaming
    constexpr int RBM = RBR > RBS ? RBR : RBS;
    constexpr int PF = (DPF == 2 || DPF == 4) ? kPF / 2 : kPF;  // register mode: W_down steps a wave holds
    constexpr int RT2 = kTile * (DPF > 0 ? RBR : RBS);  // output rows of a down item
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int nm = a.n * a.m;
    if (item >= units * T2 * ks) return;  // deduplicating kernel: a work group with no role
    const int ut = item / ks, kp = item - ut * ks;  // contraction part kp of (unit, row tile)
    const int u = ut / T2, t = ut - u * T2;
    int32_t* hcnt = a.sync + kLine * u;      // this unit's h-ready count
    int32_t* dcnt = hcnt + 1;                // this unit's finished down items
    int32_t* ocnt = a.sync + kLine * (MOE_MAX_SLOTS + t);  // arrivals on this down tile
    int e, g;
    bool sh;
    resolve(u, e, g, sh);
    // the slots' routing weights and id validity for the combine, loaded now (their
    // latency hidden behind this item's work; read after the barrier that follows
    // the arrival) so that a combining work group issues its O loads at once
    if (tid < nm) {
        const int id = a.ids[tid];
        sm.cok[tid] = (id >= 0 && id < a.N) ? 1 : 0;
        sm.cw[tid] = a.w[tid];
    }
    // ================ down: O for RT2 rows of d ================
    if (g > 0) {
        const uint32_t mat = (uint32_t)a.d * a.d_ff * F::kEsize;
        const auto rd = rsrc((SH && sh ? a.wds : a.wd) + (size_t)e * mat, mat);
        const int nslot = SH ? a.nslot : nm;
        const uint32_t hbytes = (uint32_t)nslot * a.d_ff * F::kEsize;
        const auto rh = rsrc(a.h, hbytes);
        const auto rl = rsrc(a.h + (BF16 ? hbytes : 0), hbytes);
        const auto ro = rsrc(a.O, (uint32_t)nslot * ks * a.d * 4);
        // steps kb .. ke-1 of the d_ff contraction (all of it when ks == 1), split
        // over the four waves: contiguous quarters, or with tiled weights every
        // fourth step from kb + wave
        const int S = (a.d_ff + F::kStep - 1) / F::kStep;
        const int kb = kp * S / ks, kl = (kp + 1) * S / ks - kb;
        const int s0 = TL ? kb + wave : kb + wave * kl / kWaves;
        const Steps<BF16, KF, TL ? kWaves : 1> st{
            s0, TL ? interleaved_steps(kl, wave) : kb + (wave + 1) * kl / kWaves - s0, a.d_ff, q};
        const PSteps<BF16, KF> pst{s0, st.ns, a.d_ff, a.d, q};  // W_down packed (PK)
        const TSteps tst{s0, st.ns};                           // W_down tiled (TL)
        const int ns = st.ns;
        uint32_t lrow[RBM];
#pragma unroll
        for (int rb = 0; rb < RBM; ++rb) {
            const int row = t * RT2 + rb * kTile + lr;
            const int r16 = t * RT2 / kTile + rb;  // tiled: row block (d a multiple of 16)
            lrow[rb] = TL   ? TSteps::lane_base(r16 * kTile < a.d, r16, S, lane)
                       : PK ? pst.lane_base(row < a.d, row)
                            : st.lane_base(row < a.d ? (uint32_t)row * a.d_ff * F::kEsize : kOOB);
        }
        // W_down chunk of row block rb at wave step j
        auto wload = [&](int rb, int j) {
            return TL   ? bload2<0>(rd, tst.vofs(lrow[rb], j), tst.sofs(j))
                   : PK ? bload2<0>(rd, pst.vofs(lrow[rb], j), pst.sofs(j))
                        : bload2<0>(rd, st.vofs(lrow[rb], j), st.sofs(j));
        };
        if constexpr (DPF > 0) {
            // All of this wave's W_down rows go to registers before the wait, so
            // they stream from HBM while gate/up items still run.  After the
            // wait, h is staged in LDS `gl` tokens at a time (one cooperative
            // sc1 load per chunk) and the products run from registers and LDS,
            // for any group size with one read of the weights.
            extern __shared__ __align__(16) char hs_dyn[];
            constexpr bool HSR = hs_in_red(NT * RB);
            static_assert(!HSR || sizeof(sm.red) >= kHsBudget, "h staged in the reduction array");
            char* const hs = HSR ? reinterpret_cast<char*>(&sm.red[0][0][0][0]) : hs_dyn;  // [gl][hi row, lo row], padded rows
            u32x4 pa[PF][RBR];
#pragma unroll
            for (int i = 0; i < PF; ++i)
#pragma unroll
                for (int rb = 0; rb < RBR; ++rb) pa[i][rb] = wload(rb, i);
            if (tid == 0 && !wait_count(hcnt, a.T1) && a.info) a.info[2] = MOE_E_HIP;
            __syncthreads();  // h loads (sc1) below are issued after the count was seen
            const auto rhl = rsrc(a.h, BF16 ? 2 * hbytes : hbytes);  // hi half, then lo half
            const int rowb = a.d_ff * F::kEsize + 16;      // padded LDS row
            const int tokb = BF16 ? 2 * rowb : rowb;
            const int per_row = a.d_ff * F::kEsize / 16;   // 16-byte chunks of an h row
            for (int cb = 0; cb < g; cb += a.gl) {
                const int gc = min(a.gl, g - cb);
                const int nrows = BF16 ? 2 * gc : gc;
                // kSL loads per thread in flight, then their LDS writes
                for (int c0 = 0; c0 < nrows * per_row; c0 += kSL * kThreads) {
                    u32x4 v[kSL];
                    int dst[kSL];
#pragma unroll
                    for (int j = 0; j < kSL; ++j) {
                        const int c = c0 + j * kThreads + tid;
                        uint32_t off = kOOB;
                        dst[j] = -1;
                        if (c < nrows * per_row) {
                            const int r = c / per_row, k16 = c - r * per_row;
                            const int tok = BF16 ? (r >> 1) : r, half = BF16 ? (r & 1) : 0;
                            off = (uint32_t)half * hbytes + (uint32_t)sm.grp[cb + tok] * a.d_ff * F::kEsize + k16 * 16;
                            dst[j] = tok * tokb + half * rowb + k16 * 16;
                        }
                        v[j] = bload2<kSc1>(rhl, off, 0);
                    }
#pragma unroll
                    for (int j = 0; j < kSL; ++j)
                        if (dst[j] >= 0) *reinterpret_cast<u32x4*>(hs + dst[j]) = v[j];
                }
                __syncthreads();
                const bool col_ok = lr < gc;
                const char* bp = hs + (col_ok ? lr : 0) * tokb;  // this lane's token row
                f32x4 acc[RBR];
#pragma unroll
                for (int rb = 0; rb < RBR; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    if (i < ns) {
                        const int k = st.step(i) * F::kStep + q * F::kPer;
                        const bool ok = col_ok && k < a.d_ff;
                        const u32x4 bhv = ok ? *reinterpret_cast<const u32x4*>(bp + k * F::kEsize) : zero4();
                        u32x4 blv = zero4();
                        if (BF16 && ok) blv = *reinterpret_cast<const u32x4*>(bp + rowb + k * F::kEsize);
#pragma unroll
                        for (int rb = 0; rb < RBR; ++rb) {
                            acc[rb] = F::mma(pa[i][rb], bhv, acc[rb]);
                            if (BF16) acc[rb] = F::mma(pa[i][rb], blv, acc[rb]);
                        }
                    }
                }
                static_assert(RBR <= 2 * NT * RB, "the reduction array holds 2 NT RB row blocks per wave");
                f32x4* redf = &sm.red[0][0][0][0];  // [kWaves][RBR][64]
                if constexpr (HSR) __syncthreads();  // every wave's reads of h are done before redf overwrites it
#pragma unroll
                for (int rb = 0; rb < RBR; ++rb) redf[(wave * RBR + rb) * 64 + lane] = acc[rb];
                __syncthreads();
                if (wave < RBR) {
                    const int rb = wave;
                    f32x4 v = redf[rb * 64 + lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) v += redf[(w * RBR + rb) * 64 + lane];
                    const int i0 = t * RT2 + rb * kTile + 4 * q;
                    if (col_ok && i0 < a.d)  // d % 8 == 0: rows i0..i0+3 all valid
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                                               (((uint32_t)sm.grp[cb + lr] * ks + kp) * a.d + i0) * 4, 0,
                                                               kSc1);
                    stores_complete();
                }
                __syncthreads();
            }
        } else
        for (int base = 0; base < g; base += 16 * NT) {
            u32x4 ad[P][RBS], bh[P][NT], bl[P][NT];
            uint32_t lh[NT];
            auto issue_a = [&](int slot, int j) {
#pragma unroll
                for (int rb = 0; rb < RBS; ++rb) ad[slot][rb] = wload(rb, j);
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
            for (int i = 0; i < P; ++i) {  // weights first, in slot order (see gate_up)
                issue_a(i, i);
                __builtin_amdgcn_sched_barrier(0);
            }
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
            for (int i = 0; i < P; ++i) {
                issue_b(i, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 acc[RBS][NT];
#pragma unroll
            for (int rb = 0; rb < RBS; ++rb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[rb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < ns; s += P) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int i = hh * H; i < hh * H + H; ++i)
#pragma unroll
                        for (int rb = 0; rb < RBS; ++rb)
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
            for (int rb = 0; rb < RBS; ++rb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) sm.red[wave][0][rb * NT + tt][lane] = acc[rb][tt];
            __syncthreads();
            if (wave < RBS * NT) {
                const int rb = wave / NT, tt = wave - rb * NT;
                f32x4 v = sm.red[0][0][wave][lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) v += sm.red[w][0][wave][lane];
                const int gi = base + tt * 16 + lr;
                const int i0 = t * RT2 + rb * kTile + 4 * q;
                if (gi < g && i0 < a.d)  // d % 8 == 0: rows i0..i0+3 all valid
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                                           (((uint32_t)sm.grp[gi] * ks + kp) * a.d + i0) * 4, 0, kSc1);
                stores_complete();
            }
            __syncthreads();
        }
        // the unit's last down item resets the unit's counters for the next call
        // (every down item of the unit has seen the full h-ready count by now)
        if (tid == 0 && atomicAdd(dcnt, 1) == T2 * ks - 1) {
            __hip_atomic_store(hcnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dcnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // arrival on this row tile; the last unit to arrive combines its rows
    if (tid == 0) {
        const int old = atomicAdd(ocnt, 1);  // after the writers' completed stores and the barrier
        s_last = old == units * ks - 1;
        if (s_last) __hip_atomic_store(ocnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // all arrived
    }
    __syncthreads();  // O loads (sc1) below are issued after the last arrival was seen
    if (s_last) {
        // y_t = sum_j w_tj sum_p O_(tj, p) + sum_s sum_p O_(shared s, t, p) for 4 rows
        // per thread: slots in increasing j, then shared experts in increasing s,
        // each slot's contraction parts p in increasing order (w_tj applied to each
        // part); the O loads (sc1) of up to kCJ (slot, part) pairs are in flight
        // together
        constexpr int kCJ = 8;
        const int i0 = t * RT2;
        const int q4 = min(RT2, a.d - i0) / 4;  // d % 8 == 0
        const auto rO = rsrc(a.O, (uint32_t)(SH ? a.nslot : nm) * ks * a.d * 4);
        const int nr = a.m * ks;                                  // routed (slot, part) pairs of a token
        const int npair = nr + (SH ? a.n_shared * ks : 0);        // and the shared experts' pairs
        for (int o = tid; o < a.n * q4; o += kThreads) {
            const int tok = o / q4, i = i0 + 4 * (o - tok * q4);
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c0 = 0; c0 < npair; c0 += kCJ) {
                u32x4 ov[kCJ];
                float wv[kCJ];
                bool ok[kCJ];
#pragma unroll
                for (int jj = 0; jj < kCJ; ++jj) {
                    const int c = c0 + jj;
                    int sl = -1;
                    float wgt = 1.f;
                    if (c < nr) {
                        const int s = tok * a.m + c / ks;
                        if (sm.cok[s]) {
                            sl = s;
                            wgt = sm.cw[s];
                        }
                    } else if (SH && c < npair) {
                        sl = nm + ((c - nr) / ks) * a.n + tok;
                    }
                    ok[jj] = sl >= 0;
                    wv[jj] = wgt;
                    ov[jj] = bload_sc1(rO, ok[jj] ? (((uint32_t)sl * ks + c % ks) * a.d + i) * 4 : kOOB);
                }
#pragma unroll
                for (int jj = 0; jj < kCJ; ++jj)
                    if (ok[jj])
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[jj], __uint_as_float(ov[jj][r]), acc[r]);
            }
            f32x4* yp = reinterpret_cast<f32x4*>(a.y + (size_t)tok * a.d + i);
            if (a.accumulate) acc += *yp;  // y is read only when the call accumulates
            *yp = acc;
        }
    }
}

// The per-slot kernel with 16- or 32-row down items in registers and one token tile
// holds its registers to 4 waves per SIMD, so that a small pass's gate/up and down
// work groups are all resident at once (a performance choice: every wait is on a
// lower work-group id, so no wait depends on residency); with 64-row items (half as
// many) it runs at the 3 waves their registers allow, and measured faster so.  With streaming down items (long
// d_ff) the work groups cannot all be resident anyway, and the cap (more work
// groups per compute unit, each keeping less in flight) measured slower: a
// Mixtral-shaped pass at n = 1 took 157 us against 140 us without it.  With 2 or 4
// token tiles (shared experts, n > 16) the cap made the kernel spill.  With 2 token
// tiles (passes of 17..32 tokens) the kernel is held to 3 waves per SIMD (no VGPR
// spills for whole K steps, 3-11 for a ragged K): the latency-bound down items of a
// 32-token tree pass overlap more, 6 % faster than at the 2 waves its registers
// would otherwise allow.
// RC: the remainder cut of large tiles (gate_up_groups_rc), a variant of its own.
template <bool BF16, int MODE, int NT, int RB, bool KF, int DPF, int LAY, bool SH, bool RC = false>
__global__ __launch_bounds__(kThreads, (MODE == kPerSlot && (DPF == 1 || DPF == 2) && NT == 1) ? 4 : (NT == 2 ? 3 : 1)) void k_expert(
    Args a) {
    constexpr bool TL = LAY == kLayTiled;
    // ring depth in steps: operand registers per step are (2*RB + NT) for gate/up
    // and (RB + 2*NT) for down, 4 VGPRs each
    constexpr int P = (2 * RB + NT) <= 3 ? 8 : ((2 * RB + NT) <= 6 ? 4 : 2);
    // down items: row blocks in register mode (RBR: the W_down rows a wave holds),
    // streaming RB like the gate/up items (down_work)
    constexpr int RBR = DPF == 4 ? 4 : (DPF == 2 || DPF == 3 ? 2 : 1), RBS = RB;
    __shared__ Smem<NT * RB> sm;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int nm = a.n * a.m;
    const bool want_status = a.info != nullptr && blockIdx.x == 0;

    // The pass's units and gate/up work groups.  The per-slot kernel's are the
    // host's (one unit per slot).  The deduplicating kernel's real units, one per
    // distinct expert, are known on the device only: the host sized the grid for the
    // largest pass any U up to min(n m, N) could give, and every work group counts
    // the U distinct experts (the ids are loaded once into LDS) and takes its role
    // among U routed units (at least one, so a pass without valid ids still writes
    // y) and the shared experts: gate/up shares over their tiles, then their down
    // items, and the work groups left over at the end of the grid exit.
    int units = a.units, units_r = a.units_r, g1 = a.g1;
    if (MODE == kDedup || want_status) {
        load_ids<NT * RB>(a, sm, want_status);
        int e_, g_, U;
        select_unit<NT * RB>(a, sm, -1, false, e_, g_, U, false);  // (load_ids ended with a barrier)
        U = uni(U);
        if (MODE == kDedup) {
            units_r = max(U, 1);
            units = units_r + (SH ? a.n_shared : 0);
            g1 = RC ? gate_up_groups_rc(units * a.T1, a.S1, a.split_ok, kDedupSplitUpper)
                    : gate_up_groups(units * a.T1, a.S1, a.split_ok, kDedupSplitUpper);
        }
        if (want_status && tid == 0) {
            a.info[0] = U;
            a.info[1] = sm.id_status ? MOE_E_IDS : MOE_OK;
            a.info[2] = MOE_OK;  // a bounded wait that expires later overwrites this
        }
    }
    const bool phase1 = (int)blockIdx.x < g1;
    // Down items in register mode or streaming (down_shape).  The per-slot kernel's
    // shape is the host's; the deduplicating kernel takes it for its real units (its
    // variants with DPF > 0 are those where the host found a wave's share of W_down
    // and the largest group's h fit, so register mode is allowed), streaming with
    // the host's contraction parts a.ks.
    bool reg = DPF > 0;
    int T2 = a.T2, ks = a.ks;
    if (MODE == kDedup) {
        const DownShape ds = down_shape(units, g1, a.d, DPF > 0, RBR, RBS, a.reg_wgs, a.ks);
        reg = DPF > 0 && ds.reg;
        T2 = ds.T2;
        ks = ds.ks;
    }

    // The unit u: expert e and its slots sm.grp[0..g); sh: e is a shared expert (all
    // n tokens, weight 1, slots nm + e*n + t).
    auto resolve = [&](int u, int& e, int& g, bool& sh) {
        sh = SH && u >= units_r;
        if (sh) {
            e = u - units_r;
            g = a.n;
            __syncthreads();  // the previous unit's reads of sm.grp are done
            if (tid < a.n) sm.grp[tid] = nm + e * a.n + tid;
            __syncthreads();
        } else if (MODE == kDedup) {
            int U;
            select_unit<NT * RB>(a, sm, u, true, e, g, U);
            e = uni(e);
            g = uni(g);
        } else {
            const int id = uni(a.ids[u]);
            e = (id >= 0 && id < a.N) ? id : -1;
            g = e >= 0 ? 1 : 0;
            if (tid == 0) sm.grp[0] = u;  // (gate_up ends with a barrier after its last read of sm.grp)
            __syncthreads();
        }
    };

    if (phase1) {
        // ================ gate / up: h for RT rows of d_ff per tile ================
        // The gate/up work, (unit, row tile, K step) in that order, is cut into g1
        // equal contiguous shares, one per work group; a tile cut between work
        // groups is a split tile (see gate_up).
        // Without a split, work group wi holds tile wi whole.  With one, the
        // products below stay under 2^31: at most kMaxSplitTiles tiles and
        // g1 <= kMaxSplitTiles.
        const int tiles = units * a.T1;
        const bool split = g1 != tiles;
        // RC variants, from the kernel's bound of tiles on: the remainder cut (RcPlan;
        // its arithmetic also stays under 2^31)
        const bool rcm = RC && split && tiles >= (MODE == kPerSlot ? 2 * kCUs : kDedupSplitUpper);
        const RcPlan rp(tiles, a.S1, g1);
        const int ltot = tiles * a.S1;
        const int wi = blockIdx.x;
        // (integer divisions run on the vector unit: readfirstlane keeps the
        // work-group-uniform values in scalar registers)
        // The segments run last to first: a work group's last segment is the head
        // of a split tile (it contributes without waiting) and its first is the
        // tail of one (it finalises, waiting on lower work-group ids).  In this
        // order no wait depends on another wait.
        const int lbeg = uni(rcm ? rp.lbeg(wi) : (split ? wi * ltot / g1 : wi * a.S1));
        int cur = -1, e = -1, g = 0;
        bool sh = false;
        for (int L = uni(rcm ? rp.lend(wi) : (split ? (wi + 1) * ltot / g1 : (wi + 1) * a.S1)); L > lbeg;) {
            const int tile = uni((L - 1) / a.S1);
            const int k1 = L - tile * a.S1;
            const int k0 = max(0, lbeg - tile * a.S1);
            L = tile * a.S1 + k0;
            const int u = uni(tile / a.T1), t = tile - u * a.T1;
            if (u != cur) {
                resolve(u, e, g, sh);
                cur = u;
            }
            if (g == 0) continue;
            // work groups whose shares meet this tile: first .. last
            const int first = uni(rcm ? rp.first(tile) : (split ? ((tile * a.S1 + 1) * g1 - 1) / ltot : wi));
            const int last = uni(rcm ? rp.last(tile) : (split ? ((tile * a.S1 + a.S1) * g1 - 1) / ltot : wi));
            // (a cut tile's counter: its index among the cut tiles)
            const int ctile = rcm ? (tile < rp.W ? 0 : tile - rp.W) : tile;
            const bool fin = gate_up<BF16, NT, RB, KF, P, SH, TL>(a, sm, e, sh, g, t, k0, k1, ctile,
                                                              last - first + 1, wi - first);
            if (tid == 0 && fin) atomicAdd(a.sync + kLine * u, 1);  // h-ready count of unit u
        }
    } else {
        const int item = (int)blockIdx.x - g1;
        if (MODE == kDedup && DPF > 0 && !reg)
            down_work<BF16, MODE, NT, RB, KF, 0, LAY, SH>(a, sm, s_last, item, units, T2, ks, resolve);
        else
            down_work<BF16, MODE, NT, RB, KF, DPF, LAY, SH>(a, sm, s_last, item, units, T2, ks, resolve);
    }
}

struct Plan {
    int units, units_r, nslot, T1, T2, nt, rb, ks;
    int g1, S1;  // gate/up work groups, K steps per gate/up tile
    bool split_ok;  // the workspace holds partial sums of split gate/up tiles
    size_t part_off;
    int dpf;     // down items: 0 streaming, 1, 2, 4 register mode (16, 32, 64 rows), 3 register
                 // mode (32 rows of up to kPF steps); deduplicating kernel: register mode
                 // allowed, decided on the device
    bool rc;     // gate/up tiles: the remainder cut (gate_up_groups_rc, kernel variant RC)
    int reg_wgs; // most work groups of a pass with register-mode down items
    int down_wgs;  // down work groups of the grid
    int grid;      // work groups of the launch
    int gl;      // register mode: tokens of h staged in LDS at a time
    size_t lds;  // register mode: dynamic LDS bytes
    size_t h_off, o_off, sync_off, total;
};

template <bool BF16, int MODE, int NT, int RB, int LAY, bool SH>
void launch_lay(const Args& args, const Plan& p, int grid, hipStream_t st) {
    constexpr int step = Fmt<BF16>::kStep;
    // tiled weights have K a multiple of the step in both contractions (check_desc)
    const bool kf = LAY == kLayTiled || (args.d % step == 0 && args.d_ff % step == 0);
    // the remainder cut: planned only for bf16 passes of large tiles with streaming
    // down items, one token tile and no shared experts
    if constexpr (BF16 && NT == 1 && RB == 2 && !SH) {
        if (kf && p.rc && p.dpf == 0) {
            hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 0, LAY, SH, true>), dim3(grid), dim3(kThreads), 0,
                               st, args);
            return;
        }
    }
    // 64-row register items: one token tile, or two in the deduplicating kernel
    // (groups of up to 32 tokens, staged in chunks)
    if constexpr ((NT == 1 || (NT == 2 && MODE == kDedup)) && RB == 2) {
        if (kf && p.dpf == 4) {
            hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 4, LAY, SH>), dim3(grid), dim3(kThreads), p.lds, st,
                               args);
            return;
        }
    }
    if constexpr (NT == 1 && RB == 2) {
        if (kf && p.dpf == 3) {
            hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 3, LAY, SH>), dim3(grid), dim3(kThreads), p.lds, st,
                               args);
            return;
        }
    }
    if (kf && p.dpf == 2)  // (32-row register mode is planned only for whole steps)
        hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 2, LAY, SH>), dim3(grid), dim3(kThreads), p.lds, st,
                           args);
    else if (kf && p.dpf == 1)
        hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 1, LAY, SH>), dim3(grid), dim3(kThreads), p.lds, st,
                           args);
    else if (kf)
        hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, true, 0, LAY, SH>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if constexpr (LAY != kLayTiled) {
        if (p.dpf)
            hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, false, 1, LAY, SH>), dim3(grid), dim3(kThreads), p.lds,
                               st, args);
        else
            hipLaunchKernelGGL((k_expert<BF16, MODE, NT, RB, false, 0, LAY, SH>), dim3(grid), dim3(kThreads), 0, st,
                               args);
    }
}

template <bool BF16, int MODE, int NT, int RB, bool SH>
void launch_rb(const Args& args, const Plan& p, int grid, hipStream_t st, int lay) {
    if (lay == kLayTiled) launch_lay<BF16, MODE, NT, RB, kLayTiled, SH>(args, p, grid, st);
    else if (lay == kLayPacked) launch_lay<BF16, MODE, NT, RB, kLayPacked, SH>(args, p, grid, st);
    else launch_lay<BF16, MODE, NT, RB, kLayPlain, SH>(args, p, grid, st);
}

// Kernel variant for the plan.  Shared experts (SH) are a variant of their own, so
// that passes without them carry none of their registers; a per-slot pass without
// them always takes one token column tile.
template <bool BF16, int MODE, bool SH>
void launch_nt(const Args& args, const Plan& p, int grid, hipStream_t st, int lay) {
    if constexpr (MODE == kPerSlot && !SH) {
        launch_rb<BF16, MODE, 1, 2, SH>(args, p, grid, st, lay);
    } else {
        if (p.nt == 1) launch_rb<BF16, MODE, 1, 2, SH>(args, p, grid, st, lay);
        else if (p.nt == 2) launch_rb<BF16, MODE, 2, 2, SH>(args, p, grid, st, lay);
        else launch_rb<BF16, MODE, 4, 1, SH>(args, p, grid, st, lay);
    }
}

// The launchers, one per (bf16, kernel, shared experts), each defined in its own
// compilation of expert_launch.hip; internal to the library (not exported).
using Launcher = void (*)(const Args&, const Plan&, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_0_0_0(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_0_0_1(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_0_1_0(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_0_1_1(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_1_0_0(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_1_0_1(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_1_1_0(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);
__attribute__((visibility("hidden"))) void launch_expert_1_1_1(const Args& a, const Plan& p, int grid, hipStream_t st, int lay);

}  // namespace moe_k
