// route.h -- top-K gate selection and the token -> expert dispatch.
//
// topk_kernel: one wavefront per token, a radix select.  Each logit maps to
// an order-preserving 32-bit key (NaN ranks as -inf, -0 as +0).  32
// bisection steps, each counting keys >= a candidate with one ballot per
// register, find the K-th largest key tau exactly; the selection is every
// key > tau plus the lowest-index keys == tau, which is exactly the first K
// in (larger logit, then lower expert index) order.  The K winners are
// compacted through LDS and each ranks itself against the others
// (reading them back 8 at a time).  The gates
// are the softmax over the K selected logits, which equals the full softmax
// renormalised over them.
//
// Dispatch is a stable counting sort of the T*K (token, rank) pairs by
// expert, done with per-block bit masks instead of atomics on counters:
// a block of 256 tokens marks, for every expert, which of its tokens chose
// that expert (256 bits = 4 words per expert in LDS).  The popcount of the
// mask is the block's count for the expert; the popcount of the bits below
// a token is that pair's rank inside the block.  A scan over blocks and
// experts turns these into slots.  Each token chooses an expert at most once,
// so the slots of an expert come out ordered by token: the result is
// deterministic and does not depend on scheduling.
#pragma once

#include "layer.h"

namespace lmoe {

constexpr int kRouteTok = 256;   // tokens per dispatch block
constexpr int kMaxExperts = 2048;
constexpr int kMaxK = 64;

__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) v = -INFINITY;
    if (v == 0.0f) v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(unsigned long long m) { return __popcll(m); }

// Split-reduction input of the top-K kernel: nsplit fp32 partial tiles
// part[s][T][stride] of [z | h_s | logits] (lz + m_s + N columns, rows
// padded to a multiple of 4 floats).  nsplit = 0: the logits are already in
// LayerArgs::logits (bias included), and z and a_s are written.
struct PartIn {
    const float* part;
    int nsplit, stride, lz;   // nsplit <= kMaxSplit
};
constexpr int kMaxSplit = 16;

// Top-K of token t by one wavefront, from its N logits at lg (global
// memory or LDS).  s_key / s_idx / s_val: 64 entries of LDS private to the
// calling wave (s_key and s_idx 16-byte aligned).
template <int NPL>
__device__ inline void topk_token(const LayerArgs& a, int t, const float* lg, uint32_t* s_key, int* s_idx,
                                  float* s_val) {
    const int lane = threadIdx.x & 63;
    float v[NPL];
    uint32_t key[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < a.N ? lg[e] : -INFINITY;
        key[j] = e < a.N ? order_key(v[j]) : 0u;  // padding sorts below every real key
    }
    const int K = a.K;
    // K-th largest key by bisection on its bits.  It stops early once
    // exactly K keys reach the candidate: those are the K largest, and tau =
    // cand selects them below (keys equal to tau are taken as ties).  With a
    // tie at the K-th key no count equals K and all 32 bits are resolved.
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) cnt += popc64(__ballot(key[j] >= cand));
        if (cnt >= K) tau = cand;
        if (cnt == K) break;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) gt += popc64(__ballot(key[j] > tau));
    const int need = K - gt;  // keys equal to tau still to take, lowest index first
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int eq_seen = 0, base = 0;
    // entries past the K winners: key 0, below every real key (the ranking
    // below reads the first multiple of 8 entries)
    s_key[lane] = 0u;
    s_idx[lane] = 0x7fffffff;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const bool eq = key[j] == tau;
        const unsigned long long me = __ballot(eq);
        const bool take = key[j] > tau || (eq && eq_seen + popc64(me & below) < need);
        eq_seen += popc64(me);
        const unsigned long long mt = __ballot(take);
        if (take) {
            const int pos = base + popc64(mt & below);
            s_key[pos] = key[j];
            s_idx[pos] = lane + 64 * j;
            s_val[pos] = v[j];
        }
        base += popc64(mt);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // winner `lane` ranks itself against all K winners, reading their keys
    // and indices 8 at a time (the same LDS address in every lane: one
    // broadcast read each, all of a batch in flight together)
    float my_v = -INFINITY;
    uint32_t mk = 0u;
    int my_rank = 0, my_idx = 0;
    if (lane < K) {
        mk = s_key[lane];
        my_idx = s_idx[lane];
        my_v = s_val[lane];
    }
    for (int q0 = 0; q0 < K; q0 += 8) {
        const uint4 ka = *reinterpret_cast<const uint4*>(s_key + q0);
        const uint4 kb = *reinterpret_cast<const uint4*>(s_key + q0 + 4);
        const int4 ia = *reinterpret_cast<const int4*>(s_idx + q0);
        const int4 ib = *reinterpret_cast<const int4*>(s_idx + q0 + 4);
        const uint32_t qk[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
        const int qi[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) my_rank += (qk[u] > mk || (qk[u] == mk && qi[u] < my_idx)) ? 1 : 0;
    }
    float mx = my_v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float ex = lane < K ? expf(my_v - mx) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane < K) {
        a.ids[(size_t)t * K + my_rank] = my_idx;
        a.gates[(size_t)t * K + my_rank] = ex / sum;
    }
    __builtin_amdgcn_wave_barrier();
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(LayerArgs a) {
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    __shared__ __align__(16) uint32_t s_key[4][64];
    __shared__ __align__(16) int s_idx[4][64];
    __shared__ float s_val[4][64];
    if (t >= a.T) return;
    topk_token<NPL>(a, t, a.logits + (size_t)t * a.N, s_key[wave], s_idx[wave], s_val[wave]);
}

// Two workgroups per token, after the split projection, each adding partial
// tiles in split order: blockIdx.y = 0 the logits (then the bias, into LDS),
// after which wave 0 selects the top K; blockIdx.y = 1 z and the shared
// expert's h_s (relu(h_s)^2), rounded once to bf16, to global memory.  The
// selecting workgroup thus waits only for the logits' partials.
template <int NPL>
__global__ __launch_bounds__(256) void topk_part_kernel(LayerArgs a, PartIn pin) {
    const int t = blockIdx.x;
    __shared__ float lg[64 * NPL];
    __shared__ __align__(16) uint32_t s_key[64];
    __shared__ __align__(16) int s_idx[64];
    __shared__ float s_val[64];
    const size_t ps = (size_t)a.T * pin.stride;
    const float* pt = pin.part + (size_t)t * pin.stride;
    const int le = pin.lz + a.m_s;   // first logit column
    // The partials of a value are all loaded before they are added (in split
    // order), so their latencies overlap; a thread's first two logits (or
    // first group of 4 z columns) are loaded together, so the usual sizes
    // (le <= 1024, N <= 512) take one round trip to memory.  The loads are
    // unconditional (indices past the end and splits past nsplit are clamped
    // to valid ones inside the partial rows, and their values not used):
    // conditional loads compile to branches that each wait for the loads
    // before them.
    const int s_last = pin.nsplit - 1;
    auto load_lg = [&](int e, float* v, float& b) {
        const int ec = min(e, a.N - 1);
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s) v[s] = pt[min(s, s_last) * ps + le + ec];
        b = a.bias ? a.bias[ec] : 0.0f;
    };
    auto add_lg = [&](int e, const float* v, float b) {
        if (e >= a.N) return;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < pin.nsplit) acc += v[s];
        lg[e] = a.bias ? acc + b : acc;
    };
    // z (columns [0, lz)) and the shared expert's relu(h_s)^2 (columns
    // [lz, le)), rounded once to bf16
    bf16* zo = static_cast<bf16*>(a.z_w) + (size_t)t * a.l;
    bf16* so = a.m_s > 0 ? static_cast<bf16*>(a.a_s) + (size_t)t * a.m_s - pin.lz : nullptr;
    auto load_z = [&](int c, f32x4* v) {
        // (with no z or h_s columns, le == 0, column 0 is a logit column:
        // still inside the partial row, and add_z() skips the value)
        const int cc = max(0, min(c, le - 4));
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s) v[s] = *reinterpret_cast<const f32x4*>(pt + min(s, s_last) * ps + cc);
    };
    auto add_z = [&](int c, const f32x4* v) {
        if (c >= le) return;
        f32x4 zs = v[0];
#pragma unroll
        for (int s = 1; s < kMaxSplit; ++s)
            if (s < pin.nsplit) zs += v[s];
        if (c >= pin.lz) {   // (lz is a multiple of 64: no group of 4 straddles it)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float r = zs[i] > 0.0f ? zs[i] : 0.0f;
                zs[i] = r * r;
            }
        }
        const bf16 b[4] = {(bf16)zs[0], (bf16)zs[1], (bf16)zs[2], (bf16)zs[3]};
        *reinterpret_cast<uint2*>((c < pin.lz ? zo : so) + c) = *reinterpret_cast<const uint2*>(b);
    };
    if (blockIdx.y == 1) {
        for (int c = 4 * (int)threadIdx.x; c < le; c += 1024) {
            f32x4 v[kMaxSplit];
            load_z(c, v);
            add_z(c, v);
        }
        return;
    }
    {
        float v0[kMaxSplit], v1[kMaxSplit], b0, b1;
        const int e = (int)threadIdx.x;
        load_lg(e, v0, b0);
        load_lg(e + 256, v1, b1);
        add_lg(e, v0, b0);
        add_lg(e + 256, v1, b1);
    }
    for (int e = (int)threadIdx.x + 512; e < a.N; e += 256) {
        float v[kMaxSplit], b;
        load_lg(e, v, b);
        add_lg(e, v, b);
    }
    __syncthreads();
    if (threadIdx.x < 64) topk_token<NPL>(a, t, lg, s_key, s_idx, s_val);
}

// --- dispatch helpers --------------------------------------------------------

// Mark, for every expert, which tokens of block `blk` chose it.
__device__ inline void build_masks(const LayerArgs& a, int blk, unsigned long long* masks) {
    for (int i = threadIdx.x; i < a.N * 4; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const int t0 = blk * kRouteTok;
    const int tcount = min(kRouteTok, a.T - t0);
    const int npairs = tcount * a.K;
    for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
        const int u = p / a.K;
        const int e = a.ids[(size_t)t0 * a.K + p];
        atomicOr(&masks[e * 4 + (u >> 6)], 1ull << (u & 63));
    }
    __syncthreads();
}

__device__ inline int mask_count(const unsigned long long* m) {
    return __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
}

__device__ inline int mask_below(const unsigned long long* m, int u) {
    int c = 0;
    const int w = u >> 6;
    for (int i = 0; i < w; ++i) c += __popcll(m[i]);
    const unsigned long long low = (u & 63) ? ((1ull << (u & 63)) - 1ull) : 0ull;
    return c + __popcll(m[w] & low);
}

// Exclusive scan of v[0..n) in LDS, n <= 2 * blockDim.x, blockDim.x == 1024.
// Returns the total.  wsum: 16 ints of LDS scratch.
__device__ inline int block_excl_scan(int* v, int n, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int a0 = 2 * tid < n ? v[2 * tid] : 0;
    const int a1 = 2 * tid + 1 < n ? v[2 * tid + 1] : 0;
    const int s = a0 + a1;
    int incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < 16; ++w) {
            const int c = wsum[w];
            wsum[w] = run;
            run += c;
        }
        wsum[16] = run;
    }
    __syncthreads();
    const int excl = incl - s + wsum[wave];
    if (2 * tid < n) v[2 * tid] = excl;
    if (2 * tid + 1 < n) v[2 * tid + 1] = excl + a0;
    const int total = wsum[16];
    __syncthreads();
    return total;
}

// From per-id counts in LDS `cnt`: counts, offsets, the active-expert list
// and the grouped-GEMM tile list in global memory; the exclusive offsets are
// also left in LDS `off`.  Only FFN experts (ids < n_ffn) are active or get
// tiles: the zero-computation experts' slots (the last ones) are never run.
// tmp, wsum: LDS scratch.
__device__ inline void finish_scan(const LayerArgs& a, const int* cnt, int* off, int* tmp, int* wsum) {
    const int N = a.N;
    for (int e = threadIdx.x; e < N; e += blockDim.x) {
        const int c = cnt[e];
        a.counts[e] = c;
        off[e] = c;
        tmp[e] = (c > 0 && e < a.n_ffn) ? 1 : 0;
    }
    __syncthreads();
    const int total = block_excl_scan(off, N, wsum);
    const int n_act = block_excl_scan(tmp, N, wsum);
    for (int e = threadIdx.x; e < N; e += blockDim.x) {
        a.offsets[e] = off[e];
        if (cnt[e] > 0 && e < a.n_ffn) a.active[tmp[e]] = e;
    }
    if (threadIdx.x == 0) {
        a.offsets[N] = total;
        *a.n_active = n_act;
    }
    __syncthreads();
    // The row tiles of the experts `sel` picks, `rows` rows each, into
    // list[first ...] in expert order; returns their count.
    auto emit = [&](int rows, auto sel, int2* list, int first) {
        for (int e = threadIdx.x; e < N; e += blockDim.x) tmp[e] = sel(e) ? cdiv(cnt[e], rows) : 0;
        __syncthreads();
        const int n = block_excl_scan(tmp, N, wsum);
        for (int e = threadIdx.x; e < N; e += blockDim.x) {
            const int nt = sel(e) ? cdiv(cnt[e], rows) : 0, base = first + tmp[e], o = off[e];
            for (int i = 0; i < nt; ++i) list[base + i] = make_int2(e, o + i * rows);
        }
        __syncthreads();
        return n;
    };
    auto ffn = [&](int e) { return e < a.n_ffn; };
    if (a.tall_rows == 0) {
        const int n = emit(a.tile_rows, ffn, a.tiles, 0);
        if (threadIdx.x == 0) *a.n_tiles = n;
    } else {
        // experts with at most tile_rows rows: tile_rows-row tiles; the
        // others: tall_rows-row tiles, in the second list
        auto light = [&](int e) { return e < a.n_ffn && cnt[e] <= a.tile_rows; };
        auto heavy = [&](int e) { return e < a.n_ffn && cnt[e] > a.tile_rows; };
        const int nl = emit(a.tile_rows, light, a.tiles, 0);
        const int nt = emit(a.tall_rows, heavy, a.tiles_tall, 0);
        if (threadIdx.x == 0) {
            *a.n_tiles = nl;
            *a.n_tiles_tall = nt;
        }
    }
    // the zero row of every expert-output plane (row T*K), read by the
    // combine for zero-computation experts
    if (a.N > a.n_ffn) {
        const int per_row = a.y_row_bytes / 16;
        const size_t rows = (size_t)a.T * a.K;
        for (int i = threadIdx.x; i < a.y_planes * per_row; i += blockDim.x) {
            const size_t p = (size_t)(i / per_row);
            char* row = static_cast<char*>(a.ybuf) + (p * (rows + 1) + rows) * a.y_row_bytes;
            reinterpret_cast<uint4*>(row)[i % per_row] = kZero16;
        }
    }
    __syncthreads();
}

__device__ inline void scatter_block(const LayerArgs& a, int blk, const unsigned long long* masks,
                                     const int* base_of_expert) {
    const int t0 = blk * kRouteTok;
    const int tcount = min(kRouteTok, a.T - t0);
    const int npairs = tcount * a.K;
    for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
        const int u = p / a.K;
        const int flat = t0 * a.K + p;
        const int e = a.ids[flat];
        const int slot = base_of_expert[e] + mask_below(masks + e * 4, u);
        a.perm[slot] = flat;
        a.slot_of[flat] = slot;
    }
}

// Whole dispatch in one workgroup (T <= 256 tokens).
__global__ __launch_bounds__(1024) void dispatch_one_block_kernel(LayerArgs a) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long* masks = smem_u64;                      // [N*4]
    int* cnt = reinterpret_cast<int*>(masks + a.N * 4);         // [N]
    int* off = cnt + a.N;                                       // [N]
    int* tmp = off + a.N;                                       // [N]
    int* wsum = tmp + a.N;                                      // [17]
    build_masks(a, 0, masks);
    for (int e = threadIdx.x; e < a.N; e += blockDim.x) cnt[e] = mask_count(masks + e * 4);
    __syncthreads();
    finish_scan(a, cnt, off, tmp, wsum);
    scatter_block(a, 0, masks, off);
}

// Multi-block dispatch: count -> scan -> scatter.
__global__ __launch_bounds__(1024) void dispatch_count_kernel(LayerArgs a) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long* masks = smem_u64;
    build_masks(a, blockIdx.x, masks);
    for (int e = threadIdx.x; e < a.N; e += blockDim.x)
        a.blk_counts[(size_t)blockIdx.x * a.N + e] = mask_count(masks + e * 4);
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(LayerArgs a, int nblk) {
    extern __shared__ unsigned long long smem_u64[];
    int* cnt = reinterpret_cast<int*>(smem_u64);
    int* off = cnt + a.N;
    int* tmp = off + a.N;
    int* wsum = tmp + a.N;
    // each thread scans its expert's per-block counts, 8 blocks' counts
    // loaded at a time so that their latencies overlap
    for (int e = threadIdx.x; e < a.N; e += blockDim.x) {
        int run = 0;
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = b0 + i < nblk ? a.blk_counts[(size_t)(b0 + i) * a.N + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (b0 + i < nblk) {
                    a.blk_offsets[(size_t)(b0 + i) * a.N + e] = run;
                    run += c[i];
                }
        }
        cnt[e] = run;
    }
    __syncthreads();
    finish_scan(a, cnt, off, tmp, wsum);
}

__global__ __launch_bounds__(1024) void dispatch_scatter_kernel(LayerArgs a) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long* masks = smem_u64;
    int* base = reinterpret_cast<int*>(masks + a.N * 4);
    build_masks(a, blockIdx.x, masks);
    for (int e = threadIdx.x; e < a.N; e += blockDim.x)
        base[e] = a.offsets[e] + a.blk_offsets[(size_t)blockIdx.x * a.N + e];
    __syncthreads();
    scatter_block(a, blockIdx.x, masks, base);
}

}  // namespace lmoe
