// MoE expert operation of a speculative-decoding verification pass on gfx950: the
// router, weight packing and grouping kernels, the launch planning of the fused
// expert kernel (expert_kernel.h) and the C ABI of include/moe_expert.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "expert_kernel.h"
#include "moe_expert.h"

// Workspace of moe_expert_auto_noalloc: one copy per GPU, in the code object's
// device memory.  In host code `scratch` names a host-side stand-in, not the
// device array: host code uses only the address hipGetSymbolAddress returns for
// the current device (scratch_of_current_device).
static __device__ __align__(256) char scratch[MOE_SCRATCH_BYTES];

namespace {

using namespace moe_k;

// ---------------------------------------------------------------------------
// Router: a router sends each token to m of the N experts (paper Section 1).
// Logits l_te = W_r[e] . x_t (fp32 accumulation), then per token the m largest
// logits in descending order (equal logits: lower id first) and their softmax.
// ---------------------------------------------------------------------------
constexpr int kRP = 4;      // router: loads of a wave in flight, in steps
constexpr int kRKS = 4;     // router: most parts of the d contraction

// One workgroup per 16 experts x 16 tokens x one of KS parts of the d
// contraction; the four waves split the part.  Partial logits go to
// part[ks][t][e]; the selection kernel adds the parts in order.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_router_logits(const char* __restrict__ wr, const char* __restrict__ x,
                                                            int N, int n, int d, float* __restrict__ part) {
    using F = Fmt<BF16>;
    __shared__ f32x4 red[kWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int e0 = blockIdx.x * kTile, t0 = blockIdx.y * kTile;
    const auto rw = rsrc(wr, (uint32_t)N * d * F::kEsize);
    const auto rx = rsrc(x, (uint32_t)n * d * F::kEsize);
    const int S = (d + F::kStep - 1) / F::kStep;
    const int KS = gridDim.z, ks = blockIdx.z;
    const int kb = ks * S / KS, kl = (ks + 1) * S / KS - kb;  // this part's steps
    const int s0 = kb + wave * kl / kWaves, ns = kb + (wave + 1) * kl / kWaves - s0;
    // this lane's expert row (A operand) and token column (B operand)
    const uint32_t la = e0 + lr < N ? ((uint32_t)(e0 + lr) * d + q * F::kPer) * F::kEsize : kOOB;
    const uint32_t lb = t0 + lr < n ? ((uint32_t)(t0 + lr) * d + q * F::kPer) * F::kEsize : kOOB;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < ns; i0 += kRP) {
        u32x4 a[kRP], b[kRP];
#pragma unroll
        for (int j = 0; j < kRP; ++j) {
            const int s = s0 + i0 + j;
            const bool ok = i0 + j < ns && s * F::kStep + q * F::kPer < d;  // d % 8 == 0: whole chunks
            const uint32_t so = ok ? (uint32_t)s * F::kStep * F::kEsize : 0u;
            a[j] = bload2<0>(rw, ok ? la : kOOB, so);
            b[j] = bload2<0>(rx, ok ? lb : kOOB, so);
        }
#pragma unroll
        for (int j = 0; j < kRP; ++j) acc = F::mma(a[j], b[j], acc);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const f32x4 v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        // lane l holds experts e0 + 4*(l/16) + i for token t0 + l%16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + 4 * q + i, t = t0 + lr;
            if (e < N && t < n) part[((size_t)ks * n + t) * N + e] = v[i];
        }
    }
}

// (v, id) beats (w, jd): larger logit, or equal logits and lower id
__device__ __forceinline__ bool rk_before(float v, int id, float w, int jd) { return v > w || (v == w && id < jd); }

// One wave per token (four per workgroup, no barriers): the logits (the KS parts
// added in order, written out), each lane holding experts lane + 64 j; m rounds of
// a wave-wide selection of the best remaining (logit, id); the softmax of the m
// selected logits.
constexpr int kRPerLane = MOE_MAX_EXPERTS / 64;

__global__ __launch_bounds__(kThreads) void k_router_topm(const float* __restrict__ part, int KS, int n, int N, int m,
                                                          float* __restrict__ logits, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
    __shared__ float selv[kWaves][MOE_MAX_SLOTS];
    __shared__ int seli[kWaves][MOE_MAX_SLOTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * kWaves + wave;
    if (t >= n) return;  // whole waves; the kernel has no barrier
    // every (expert, part) load of the lane in flight at once (out-of-range ones
    // read zero through the descriptor, no branches), then the sums in part order
    const auto rp = rsrc(part, (uint32_t)KS * n * N * 4);
    float pv[kRPerLane][kRKS];
#pragma unroll
    for (int j = 0; j < kRPerLane; ++j)
#pragma unroll
        for (int ks = 0; ks < kRKS; ++ks) {
            const int e = lane + 64 * j;
            const bool ok = e < N && ks < KS;
            pv[j][ks] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rp, ok ? (((uint32_t)ks * n + t) * N + e) * 4u : kOOB, 0, 0));
        }
    float v[kRPerLane];
#pragma unroll
    for (int j = 0; j < kRPerLane; ++j) {
        float s = pv[j][0];
#pragma unroll
        for (int ks = 1; ks < kRKS; ++ks)
            if (ks < KS) s += pv[j][ks];
        v[j] = s;
        const int e = lane + 64 * j;
        if (e < N) logits[(size_t)t * N + e] = s;
    }
    uint32_t taken = 0u;  // bit j: expert lane + 64 j already selected
    for (int r = 0; r < m; ++r) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kRPerLane; ++j) {
            const int e = lane + 64 * j;
            if (e < N && !((taken >> j) & 1u) && rk_before(v[j], e, bv, bi)) {
                bv = v[j];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (rk_before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        // every lane now holds the winner; no candidate (only non-finite logits
        // left) gives id -1, which the expert calls skip
        if ((unsigned)bi >= (unsigned)N) bi = -1;
        else if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == 0) {
            selv[wave][r] = bv;
            seli[wave][r] = bi;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // softmax over the selected logits, the largest first; the wave's sum by a fixed
    // tree, lane 0's result for all
    const float top = selv[wave][0];
    float part_sum = 0.f;
    for (int j = lane; j < m; j += 64) part_sum += expf(selv[wave][j] - top);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part_sum += __shfl_xor(part_sum, o, 64);
    part_sum = __shfl(part_sum, 0, 64);  // one denominator for every lane
    for (int j = lane; j < m; j += 64) {
        ids[(size_t)t * m + j] = seli[wave][j];
        w[(size_t)t * m + j] = expf(selv[wave][j] - top) / part_sum;
    }
}

// Selection by rank for up to kRRMaxN experts: one workgroup of 16 waves per 16
// tokens loads their logits (the KS parts added in order, written out) into LDS and
// ranks every (token, expert) by the number of experts that come before it (larger
// logit, or equal logit and lower id): the rank is the expert's position, so the
// ranks below m are the selection, in order.  One wave per token then takes the
// softmax of the selected logits.  No rounds: the cost does not grow with m.
constexpr int kRRW = 16;                 // waves of the ranking workgroup
constexpr int kRRMaxN = 256, kRRMaxM = 64;

__global__ __launch_bounds__(64 * kRRW) void k_router_rank(const float* __restrict__ part, int KS, int n, int N, int m,
                                                           float* __restrict__ logits, int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
    __shared__ float lgt[kTile][kRRMaxN];
    __shared__ float selv[kTile][kRRMaxM];
    __shared__ int seli[kTile][kRRMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kTile;
    const int nt = min(kTile, n - t0);
    const auto rp = rsrc(part, (uint32_t)KS * n * N * 4);
    for (int it = tid; it < nt * N; it += 64 * kRRW) {
        const int t = it / N, e = it - t * N;
        float pv[kRKS];  // every part's load in flight, then the sum in part order
#pragma unroll
        for (int ks = 0; ks < kRKS; ++ks)
            pv[ks] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rp, ks < KS ? (((uint32_t)ks * n + t0 + t) * N + e) * 4u : kOOB, 0, 0));
        float v = pv[0];
#pragma unroll
        for (int ks = 1; ks < kRKS; ++ks)
            if (ks < KS) v += pv[ks];
        lgt[t][e] = v;
        logits[(size_t)(t0 + t) * N + e] = v;
    }
    __syncthreads();
    for (int it = tid; it < nt * N; it += 64 * kRRW) {
        const int t = it / N, e = it - t * N;
        const float v = lgt[t][e];
        int rank = 0;
        for (int k = 0; k < N; ++k) rank += rk_before(lgt[t][k], k, v, e) ? 1 : 0;
        if (rank < m) {
            selv[t][rank] = v;
            seli[t][rank] = e;
        }
    }
    __syncthreads();
    if (wave < nt) {  // softmax of the selected logits, the largest first; lane 0's sum for all
        const int t = wave;
        const float top = selv[t][0];
        float sum = lane < m ? expf(selv[t][lane] - top) : 0.f;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
        sum = __shfl(sum, 0, 64);
        if (lane < m) {
            ids[(size_t)(t0 + t) * m + lane] = seli[t][lane];
            w[(size_t)(t0 + t) * m + lane] = expf(selv[t][lane] - top) / sum;
        }
    }
}

// Packing of W_down into blocks of 8 columns: dst[e][c][i][k] = src[e][i][8c + k].
// One thread per 16-byte piece of a source row (8 bf16 or 4 fp32 elements).
__global__ __launch_bounds__(256) void k_pack_wdown(const char* __restrict__ src, char* __restrict__ dst, int64_t N,
                                                   int d, int d_ff, int es) {
    const int per = 16 / es;
    const int64_t prow = d_ff / per;  // pieces per source row
    const int64_t pieces = N * d * prow;
    for (int64_t gi = blockIdx.x * 256ll + threadIdx.x; gi < pieces; gi += (int64_t)gridDim.x * 256) {
        const int64_t row = gi / prow;  // e*d + i
        const int f = (int)(gi - row * prow) * per;
        const int64_t e = row / d;
        const int i = (int)(row - e * d);
        const int64_t so = (row * d_ff + f) * es;
        const int64_t dofs = (((e * (d_ff / 8) + f / 8) * d + i) * 8 + f % 8) * es;
        *reinterpret_cast<u32x4*>(dst + dofs) = *reinterpret_cast<const u32x4*>(src + so);
    }
}

// Tiled copy of E matrices [R][K] (element size es; R a multiple of 16, K of the
// 64-byte step): destination piece p (16 bytes) is lane l = p % 64 of block p / 64 =
// (e, r16, s) in that order, row r16*16 + l%16, columns s*step + (l/16)*(16/es) on.
// Writes are contiguous; each thread reads one 16-byte piece of a source row.
__global__ __launch_bounds__(256) void k_pack_tiled(const char* __restrict__ src, char* __restrict__ dst, int64_t E,
                                                   int R, int K, int es) {
    const int per = 16 / es, step = 64 / es;
    const int S = K / step, R16 = R / 16;
    const int64_t pieces = E * R16 * S * 64;
    for (int64_t p = blockIdx.x * 256ll + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * 256) {
        const int l = (int)(p & 63);
        const int64_t blk = p >> 6;
        const int s = (int)(blk % S);
        const int64_t rest = blk / S;
        const int r16 = (int)(rest % R16);
        const int64_t e = rest / R16;
        const int64_t so = ((e * R + r16 * 16 + (l & 15)) * K + (int64_t)s * step + (l >> 4) * per) * es;
        *reinterpret_cast<u32x4*>(dst + p * 16) = *reinterpret_cast<const u32x4*>(src + so);
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
    if (d->flags & ~(MOE_FLAG_ACCUMULATE | MOE_FLAG_WDOWN_PACKED | MOE_FLAG_TILED)) return MOE_E_INVAL;
    const int64_t es = d->dtype == MOE_BF16 ? 2 : 4;
    // tiled weights: one layout of all three matrices, both contractions whole steps
    if (d->flags & MOE_FLAG_TILED) {
        if (d->flags & MOE_FLAG_WDOWN_PACKED) return MOE_E_INVAL;
        if (d->d_model % (64 / es) || d->d_ff % (64 / es)) return MOE_E_INVAL;
    }
    // one expert matrix must be addressable by a 31-bit buffer offset
    if ((int64_t)d->d_model * d->d_ff * es > (1ll << 31) - 4096) return MOE_E_INVAL;
    if ((d->d_model + kTile - 1) / kTile > kMaxDownTiles) return MOE_E_INVAL;  // d_model <= 16384
    // shared experts: one counter line per unit, and h and O rows addressable by a
    // 31-bit buffer offset
    if (d->n_shared < 0 || d->n_shared > MOE_MAX_SHARED) return MOE_E_INVAL;
    if ((int64_t)n * d->m + d->n_shared > MOE_MAX_SLOTS) return MOE_E_INVAL;
    const int64_t nslot = (int64_t)n * d->m + (int64_t)d->n_shared * n;
    if (nslot * d->d_ff * 4 > (1ll << 31) - 4096 || nslot * kMaxKs * d->d_model * 4 > (1ll << 31) - 4096)
        return MOE_E_INVAL;
    return MOE_OK;
}


// work groups per compute unit at once: the per-slot register-mode kernel's launch
// bound, and what the deduplicating kernel's registers allow
constexpr int kResidentSlot = 4, kResidentDedup = 3;
// per-slot passes with shared experts: LDS for the shared experts' h chunks
constexpr int kHsBudgetShared = 12 * 1024;

Plan plan_for(const moe_layer_desc* d, int32_t n, int kind) {
    Plan p;
    const int nm = n * d->m;
    // routed units, then one unit per shared expert (all n tokens)
    p.units_r = kind == MOE_KIND_SLOT ? nm : (nm < d->N ? nm : d->N);
    p.units = p.units_r + d->n_shared;
    p.nslot = nm + d->n_shared * n;
    // token columns per MFMA pass: a group of up to 16 tokens is one column tile;
    // larger groups (dedup, or a shared expert's n tokens) take 2 or 4 so that each
    // expert is still read once
    const bool wide = kind == MOE_KIND_DEDUP || d->n_shared > 0;
    p.nt = (!wide || n <= 16) ? 1 : (n <= 32 ? 2 : 4);
    p.rb = p.nt == 4 ? 1 : 2;  // rows per item = 16 * rb; row blocks x token tiles <= 4
    p.T1 = (d->d_ff + kTile * p.rb - 1) / (kTile * p.rb);
    const bool bf = d->dtype == MOE_BF16;
    const int es = bf ? 2 : 4, step = 64 / es;  // bytes per element, elements per K step
    // Gate/up work is cut into kCUs equal shares when there are between half the
    // compute units and an upper bound of tiles (2 kCUs per-slot, kDedupSplitUpper
    // deduplicating): then no compute unit holds two tiles while another holds one.
    // With fewer tiles than half the compute units (a pass of one or two experts),
    // every tile is cut in two, so twice as many compute units stream (a compute
    // unit's own stream is bounded by the loads it keeps in flight).  Each share is
    // at least half a tile, so a tile is shared by at most kMaxContrib work groups.
    // Otherwise one work group per tile (with more tiles, cutting them measured
    // slower than the imbalance).
    // (gate_up_groups; the deduplicating kernel applies the same rule on the device
    // to its real units, U of the min(n m, N) planned here, and may cut tiles where
    // this plan does not: its workspace always holds the partial sums)
    // Large tiles (kCutMinS1 K steps or more: the Mixtral shape's 512 KB tiles) with
    // streaming down items take the remainder cut instead above the bound
    // (gate_up_groups_rc: whole rounds of kCUs tiles, the remainder cut into shares),
    // in a kernel variant of its own; bf16, one token tile, no shared experts.
    p.S1 = (d->d_model + step - 1) / step;
    const int64_t tiles = (int64_t)p.units * p.T1;
    const int64_t part_bytes = (int64_t)kMaxContrib * p.nslot * d->d_ff * 8;
    p.split_ok = part_bytes <= (64ll << 20);
    const int s2 = (d->d_ff + step - 1) / step;
    const int wsteps = (s2 + kWaves - 1) / kWaves;  // a wave's share of the down contraction
    const bool kf = d->d_model % step == 0 && d->d_ff % step == 0;
    p.rc = bf && kf && p.nt == 1 && p.rb == 2 && d->n_shared == 0 && p.S1 >= kCutMinS1 && wsteps > kPF &&
           p.split_ok;
    const int upper = kind == MOE_KIND_SLOT ? 2 * kCUs : kDedupSplitUpper;
    auto groups = [&](int t) {
        return p.rc ? gate_up_groups_rc(t, p.S1, p.split_ok, upper) : gate_up_groups(t, p.S1, p.split_ok, upper);
    };
    p.g1 = groups((int)tiles);
    const bool split = p.g1 != tiles;
    // Down items in register mode: when a wave's share of the down contraction fits
    // kPF steps and one token's h fits the LDS staging budget, and the pass's work
    // groups (gate/up, then register-mode down items) fill at most 11/4 rounds of
    // what the compute units hold at once.  h is staged gl tokens at a time (at most
    // 16, one MFMA column tile); a larger group runs its chunks one after another
    // on the same W_down registers (h loads, products, O stores in series).  A
    // per-slot pass stages one token (its shared experts' n tokens in chunks of what
    // kHsBudgetShared holds); a deduplicating pass up to what kHsBudget holds.
    // Same-box, the 32-node tree on the Qwen3 shape (groups of up to 32 tokens, two
    // token tiles): 64-row register items 146 us per pass against 164 us streaming
    // (32-row register items: 167 us); the DeepSeek-V2-Lite shape's dedup passes at
    // n = 6..8, which now stage 5 tokens a chunk, are unchanged.
    // Register-mode items prefetch their W_down while they wait, which pays for those
    // resident during gate/up; items dispatched after it run in rounds of short,
    // latency-bound work, where streaming items (twice the rows, a load ring) do
    // better.  Same-box: every pass measured at 2.7 rounds or fewer was faster in
    // register mode, every one at 3 or more faster streaming; this holds for
    // register-mode items of 16 rows, while items of 32 rows (a wave's share at most
    // kPF / 2 steps) are taken at any round count (down_shape).  The deduplicating
    // kernel counts its rounds on the device, over its real units (the U distinct
    // experts are not known here): its launch carries both forms of down item and the
    // grid covers the larger.
    const int per_tok = (d->d_ff * es + 16) * (bf ? 2 : 1);  // staged bytes per token
    const int gmax = kind == MOE_KIND_SLOT ? 1 : n;  // routed group size is at most n (valid ids)
    const int64_t resident = (int64_t)kCUs * (kind == MOE_KIND_SLOT ? kResidentSlot : kResidentDedup);
    // row blocks of a register-mode item: 64 rows (a wave's share at most kPF / 2
    // steps; one token tile, or two in the deduplicating kernel) or, deduplicating,
    // 32 rows of up to kPF steps for the one-token-tile variants; else 32 or 16 rows
    const bool wide_reg = kf && p.nt == 1 && p.rb == 2;
    const bool reg64 = wide_reg || (kf && p.nt == 2 && p.rb == 2 && kind == MOE_KIND_DEDUP);
    const int reg_rows = (kf && wsteps <= kPF / 2) ? (reg64 ? 4 : 2) : (wide_reg && kind == MOE_KIND_DEDUP ? 2 : 1);
    const int reg_dpf = reg_rows == 4 ? 4 : (reg_rows == 2 ? (wsteps <= kPF / 2 ? 2 : 3) : 1);
    p.reg_wgs = (int)(11 * resident / 4);  // (resident is a multiple of 4)
    bool reg_allowed;
    if (kind == MOE_KIND_SLOT && d->n_shared > 0) {
        const int cap = (int)std::max<int64_t>(1, kHsBudgetShared / per_tok);
        reg_allowed = wsteps <= kPF && (int64_t)per_tok <= kHsBudget;
        p.gl = reg_allowed ? std::min(n, std::min(cap, 16)) : 0;
    } else {
        const int cap = (int)std::max<int64_t>(1, kHsBudget / per_tok);
        reg_allowed = wsteps <= kPF && (int64_t)per_tok <= kHsBudget;
        p.gl = reg_allowed ? std::min(gmax, std::min(cap, 16)) : 0;
    }
    // Streaming down items (not register mode) each stream their rows' W_down after
    // the wait, at what one work group keeps in flight; with fewer than 4 items per
    // compute unit the d_ff contraction of each (unit, row tile) is cut into ks
    // parts, one item each, summed in the combine.  For the deduplicating kernel the
    // parts are counted over the planned units, min(n m, N) routed: counted over its
    // real units instead (more parts when fewer experts are distinct), the same-box
    // bench was 7 us slower on the DeepSeek-V2-Lite shape at n = 4 (correlated),
    // 5-7 us on the Mixtral shape at n = 4..8 (uniform), 6 us faster only on the
    // Mixtral shape at n = 2 (correlated).
    const int t2s = (d->d_model + kTile * p.rb - 1) / (kTile * p.rb);
    const int64_t ditems = (int64_t)p.units * t2s;
    const int ks_s = (int)std::min<int64_t>(kMaxKs, std::max<int64_t>(1, (4 * kCUs + ditems - 1) / ditems));
    const DownShape ds = down_shape(p.units, p.g1, d->d_model, reg_allowed, reg_rows, p.rb, p.reg_wgs, ks_s);
    p.T2 = ds.T2;
    p.ks = ds.ks;
    if (kind == MOE_KIND_SLOT) {
        p.dpf = ds.reg ? reg_dpf : 0;
        p.down_wgs = p.units * p.T2 * p.ks;
        p.grid = p.g1 + p.down_wgs;
    } else {
        // the device takes the shape for the U distinct experts it finds; the grid
        // covers the largest pass, gate/up and down work groups, over every U
        p.dpf = reg_allowed ? reg_dpf : 0;
        p.grid = 0;
        bool streams = false;
        for (int U = 1; U <= p.units_r; ++U) {
            const int units = U + d->n_shared;
            const int g1 = groups(units * p.T1);
            const DownShape du = down_shape(units, g1, d->d_model, reg_allowed, reg_rows, p.rb, p.reg_wgs, ks_s);
            p.grid = std::max(p.grid, g1 + units * du.T2 * du.ks);
            streams |= !du.reg;
        }
        p.down_wgs = p.grid - p.g1;
        p.ks = streams ? ks_s : 1;  // O holds the streaming form's parts if it may stream
    }
    if (!p.dpf) p.gl = 0;
    // (h staged in the reduction array when it holds kHsBudget: no dynamic LDS)
    p.lds = (p.dpf && !hs_in_red(p.nt * p.rb)) ? (size_t)p.gl * per_tok : 0;
    p.sync_off = 0;
    p.h_off = (size_t)kSyncWords * 4;
    p.o_off = p.h_off + align_up((size_t)p.nslot * d->d_ff * 4);
    p.part_off = p.o_off + align_up((size_t)p.nslot * p.ks * d->d_model * 4);
    p.total = p.part_off + ((split || (kind == MOE_KIND_DEDUP && p.split_ok)) ? align_up((size_t)part_bytes) : 0);
    return p;
}

// Zeroes `words` int32 words (the counter area at the start of a workspace).
__global__ __launch_bounds__(256) void k_zero_words(int32_t* __restrict__ p, int words) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < words; i += gridDim.x * 256) p[i] = 0;
}

template <int MODE>
int run_expert(const moe_layer_desc* d, const moe_layer_weights* W, const void* x, const int32_t* ids,
               const float* w, int32_t n, float* y, int32_t* info, void* ws, size_t ws_bytes, void* stream,
               void* const* events, int32_t n_events, bool clear_counters = false) {
    int rc = check_desc(d, n);
    if (rc != MOE_OK) return rc;
    if (!W || !W->w_gate || !W->w_up || !W->w_down || !x || !ids || !w || !y || !ws) return MOE_E_INVAL;
    if (!aligned16(W->w_gate) || !aligned16(W->w_up) || !aligned16(W->w_down) || !aligned16(x) || !aligned16(y))
        return MOE_E_INVAL;
    if (d->n_shared > 0 && (!W->w_gate_shared || !W->w_up_shared || !W->w_down_shared ||
                            !aligned16(W->w_gate_shared) || !aligned16(W->w_up_shared) || !aligned16(W->w_down_shared)))
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
    args.wgs = reinterpret_cast<const char*>(d->n_shared > 0 ? W->w_gate_shared : nullptr);
    args.wus = reinterpret_cast<const char*>(d->n_shared > 0 ? W->w_up_shared : nullptr);
    args.wds = reinterpret_cast<const char*>(d->n_shared > 0 ? W->w_down_shared : nullptr);
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
    args.units_r = p.units_r;
    args.n_shared = d->n_shared;
    args.nslot = p.nslot;
    args.T1 = p.T1;
    args.T2 = p.T2;
    args.ks = p.ks;
    args.accumulate = (d->flags & MOE_FLAG_ACCUMULATE) ? 1 : 0;
    args.gl = p.gl;
    args.g1 = p.g1;
    args.S1 = p.S1;
    args.split_ok = p.split_ok ? 1 : 0;
    args.reg_wgs = p.reg_wgs;
    args.part = reinterpret_cast<float*>(wsb + p.part_off);
    const int grid = p.grid;
    (void)hipGetLastError();
    if (clear_counters)  // a workspace whose counters may not be zero (a shared array): clear them first
        hipLaunchKernelGGL(k_zero_words, dim3((kSyncWords + 255) / 256), dim3(256), 0, st,
                           reinterpret_cast<int32_t*>(wsb + p.sync_off), kSyncWords);
    if (events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[0]), st);
    const bool bf = d->dtype == MOE_BF16;
    const int lay = (d->flags & MOE_FLAG_TILED) ? kLayTiled : (d->flags & MOE_FLAG_WDOWN_PACKED) ? kLayPacked : kLayPlain;
    const bool sh = d->n_shared > 0;
    static const Launcher launchers[2][2][2] = {  // [bf16][kernel][shared experts]
        {{launch_expert_0_0_0, launch_expert_0_0_1}, {launch_expert_0_1_0, launch_expert_0_1_1}},
        {{launch_expert_1_0_0, launch_expert_1_0_1}, {launch_expert_1_1_0, launch_expert_1_1_1}}};
    launchers[bf ? 1 : 0][MODE][sh ? 1 : 0](args, p, grid, st, lay);
    if (events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[1]), st);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

// parts of the router's d contraction: about kCUs workgroups, at least one step per wave
int router_ks(const moe_layer_desc* d, int32_t n) {
    const int wg = ((d->N + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
    const int steps = (d->d_model + (d->dtype == MOE_BF16 ? 32 : 16) - 1) / (d->dtype == MOE_BF16 ? 32 : 16);
    return std::max(1, std::min(std::min(kRKS, kCUs / wg), steps / kWaves));
}

// ---------------------------------------------------------------------------
// moe_expert_auto_noalloc: the scratch array's device address, once per device
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_E_HIP;
    if (stream) {  // the array used is the current device's: the stream must be on it
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_E_HIP;
        if ((int)sdev != dev) return MOE_E_INVAL;
    }
    if (dev >= kMaxDevices) return MOE_E_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_E_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

int router_check(const moe_layer_desc* desc, int32_t n) {
    if (!desc) return MOE_E_INVAL;
    if (desc->dtype != MOE_F32 && desc->dtype != MOE_BF16) return MOE_E_DTYPE;
    if (desc->d_model < 8 || desc->d_model % 8) return MOE_E_DTYPE;
    if (desc->N < 1 || desc->N > MOE_MAX_EXPERTS || desc->m < 1 || desc->m > desc->N || desc->m > MOE_MAX_SLOTS)
        return MOE_E_INVAL;
    if (n < 1 || n > MOE_MAX_TOKENS) return MOE_E_INVAL;
    const int64_t es = desc->dtype == MOE_BF16 ? 2 : 4;
    if ((int64_t)desc->N * desc->d_model * es > (1ll << 31) - 4096) return MOE_E_INVAL;
    return MOE_OK;
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
    size_t total = 0;  // largest over 1..n tokens (the split partial sums are not monotone in n)
    for (int32_t k = 1; k <= n; ++k) {
        const size_t t = plan_for(desc, k, kind).total;
        total = t > total ? t : total;
    }
    return total;
}

int moe_pack_w_down(const moe_layer_desc* desc, const void* w_down, void* w_down_packed, void* hip_stream) {
    if (!desc) return MOE_E_INVAL;
    moe_layer_desc dd = *desc;
    dd.flags = 0;
    dd.n_shared = 0;
    const int rc = check_desc(&dd, 1);
    if (rc != MOE_OK) return rc;
    if (!w_down || !w_down_packed || !aligned16(w_down) || !aligned16(w_down_packed)) return MOE_E_INVAL;
    const int64_t es = desc->dtype == MOE_BF16 ? 2 : 4;
    const int64_t bytes = (int64_t)desc->N * desc->d_model * desc->d_ff * es;
    const char* a0 = reinterpret_cast<const char*>(w_down);
    const char* b0 = reinterpret_cast<const char*>(w_down_packed);
    if (a0 < b0 + bytes && b0 < a0 + bytes) return MOE_E_INVAL;  // overlapping
    const int64_t pieces = bytes / 16;
    const int grid = (int)std::min<int64_t>((pieces + 255) / 256, 65536);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_pack_wdown, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream),
                       reinterpret_cast<const char*>(w_down), reinterpret_cast<char*>(w_down_packed),
                       (int64_t)desc->N, desc->d_model, desc->d_ff, (int)es);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_pack_tiled(const moe_layer_desc* desc, const void* w, void* w_tiled, int32_t mat, void* hip_stream) {
    if (!desc || (mat != MOE_MAT_GATE_UP && mat != MOE_MAT_DOWN)) return MOE_E_INVAL;
    moe_layer_desc dd = *desc;
    dd.flags = MOE_FLAG_TILED;
    dd.n_shared = 0;
    const int rc = check_desc(&dd, 1);
    if (rc != MOE_OK) return rc;
    if (!w || !w_tiled || !aligned16(w) || !aligned16(w_tiled)) return MOE_E_INVAL;
    const int64_t es = desc->dtype == MOE_BF16 ? 2 : 4;
    const int64_t bytes = (int64_t)desc->N * desc->d_model * desc->d_ff * es;
    const char* a0 = reinterpret_cast<const char*>(w);
    const char* b0 = reinterpret_cast<const char*>(w_tiled);
    if (a0 < b0 + bytes && b0 < a0 + bytes) return MOE_E_INVAL;  // overlapping
    const int R = mat == MOE_MAT_GATE_UP ? desc->d_ff : desc->d_model;
    const int K = mat == MOE_MAT_GATE_UP ? desc->d_model : desc->d_ff;
    const int64_t pieces = bytes / 16;
    const int grid = (int)std::min<int64_t>((pieces + 255) / 256, 65536);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_pack_tiled, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream), a0,
                       reinterpret_cast<char*>(w_tiled), (int64_t)desc->N, R, K, (int)es);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

size_t moe_router_workspace_bytes(const moe_layer_desc* desc, int32_t n) {
    if (router_check(desc, n) != MOE_OK) return 0;
    size_t total = 0;  // largest over 1..n tokens
    for (int32_t k = 1; k <= n; ++k)
        total = std::max(total, (size_t)router_ks(desc, k) * k * desc->N * 4);
    return total;
}

int moe_router_topk(const moe_layer_desc* desc, const void* w_router, const void* x, int32_t n,
                               float* logits, int32_t* ids, float* w, void* ws, size_t ws_bytes, void* hip_stream) {
    const int rc = router_check(desc, n);
    if (rc != MOE_OK) return rc;
    if (!w_router || !x || !logits || !ids || !w || !ws) return MOE_E_INVAL;
    if (!aligned16(w_router) || !aligned16(x) || (reinterpret_cast<uintptr_t>(logits) & 3u) ||
        (reinterpret_cast<uintptr_t>(ws) & 3u))
        return MOE_E_INVAL;
    const int KS = router_ks(desc, n);
    if (ws_bytes < (size_t)KS * n * desc->N * 4) return MOE_E_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    float* part = reinterpret_cast<float*>(ws);
    const dim3 g1((desc->N + kTile - 1) / kTile, (n + kTile - 1) / kTile, KS);
    (void)hipGetLastError();
    if (desc->dtype == MOE_BF16)
        hipLaunchKernelGGL(k_router_logits<true>, g1, dim3(kThreads), 0, st, reinterpret_cast<const char*>(w_router),
                           reinterpret_cast<const char*>(x), desc->N, n, desc->d_model, part);
    else
        hipLaunchKernelGGL(k_router_logits<false>, g1, dim3(kThreads), 0, st, reinterpret_cast<const char*>(w_router),
                           reinterpret_cast<const char*>(x), desc->N, n, desc->d_model, part);
    if (desc->N <= kRRMaxN && desc->m <= kRRMaxM)
        hipLaunchKernelGGL(k_router_rank, dim3((n + kTile - 1) / kTile), dim3(64 * kRRW), 0, st, part, KS, n, desc->N,
                           desc->m, logits, ids, w);
    else
        hipLaunchKernelGGL(k_router_topm, dim3((n + kWaves - 1) / kWaves), dim3(kThreads), 0, st, part, KS, n,
                           desc->N, desc->m, logits, ids, w);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
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

int moe_expert_auto(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x, const int32_t* ids,
                    const float* w, int32_t n, float* y, int32_t* info, void* ws, size_t ws_bytes, int32_t crossover,
                    int32_t* kind_out, void* hip_stream) {
    if (crossover < 0) return MOE_E_INVAL;
    const bool dedup = crossover > 0 && n >= crossover;
    const int rc = dedup ? run_expert<kDedup>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, nullptr, 0)
                         : run_expert<kPerSlot>(desc, weights, x, ids, w, n, y, info, ws, ws_bytes, hip_stream, nullptr,
                                                0);
    if (rc == MOE_OK && kind_out) *kind_out = dedup ? MOE_KIND_DEDUP : MOE_KIND_SLOT;
    return rc;
}

int moe_expert_auto_noalloc(const moe_layer_desc* desc, const moe_layer_weights* weights, const void* x,
                            const int32_t* ids, const float* w, int32_t n, float* y, int32_t* info,
                            int32_t crossover, int32_t* kind_out, void* hip_stream) {
    if (crossover < 0) return MOE_E_INVAL;
    int rc = check_desc(desc, n);
    if (rc != MOE_OK) return rc;
    const bool dedup = crossover > 0 && n >= crossover;
    if (plan_for(desc, n, dedup ? MOE_KIND_DEDUP : MOE_KIND_SLOT).total > (size_t)MOE_SCRATCH_BYTES)
        return MOE_E_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    void* ws = nullptr;
    rc = scratch_of_current_device(st, &ws);
    if (rc != MOE_OK) return rc;
    // the expert call validates every argument, then clears the array's counter
    // words (a kernel on the same stream) and launches
    rc = dedup ? run_expert<kDedup>(desc, weights, x, ids, w, n, y, info, ws, MOE_SCRATCH_BYTES, hip_stream, nullptr, 0,
                                    true)
               : run_expert<kPerSlot>(desc, weights, x, ids, w, n, y, info, ws, MOE_SCRATCH_BYTES, hip_stream,
                                      nullptr, 0, true);
    if (rc == MOE_OK && kind_out) *kind_out = dedup ? MOE_KIND_DEDUP : MOE_KIND_SLOT;
    return rc;
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
