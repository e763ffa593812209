// gemm2.h -- the large-tile bf16 MFMA GEMM used by the tiled path.
//
// C[r, c] = epilogue(sum_k A[r, k] * B[c, k]) over a LayerArgs problem
// (layer.h), A rows = tokens or slots, B rows = weight rows.
//
// Tile BM x BN x 64 with 256 threads as 2 x 2 waves; a wave owns
// (BM/2) x (BN/2) outputs as 32 x 32 blocks of v_mfma_f32_32x32x16_bf16.
// The weight fragment is the MFMA's first operand, so a lane's 16
// accumulators of a block are 4 groups of 4 consecutive output columns of
// one row: the epilogue reads per-row data (gate, token, residual row) once
// per lane and stores 4 columns at a time.
//
// Pipeline: global -> registers two k-tiles ahead, registers -> LDS one
// k-tile ahead (two LDS buffers).  In MFMA groups 0 and 1 of a k-tile,
// group g writes parts 2g and 2g+1 of the next k-tile to LDS and then loads
// the same parts of the k-tile after it into the freed registers, so each
// load is at least two groups old when the next k-tile starts.  LDS rows are 64 bf16 = 8
// units of 16 bytes; unit c of row r is stored at c ^ (r & 7), so the
// 16-byte reads of 8 consecutive rows hit distinct bank groups.
//
// The grid is one-dimensional.  Consecutive workgroup ids go to different
// XCDs (round robin over 8), so ids are remapped such that each XCD gets a
// contiguous range of logical tiles; logical tiles run row-tile-major, so
// the tiles of one expert (its rows x all column tiles) share one XCD's L2.
#pragma once

#include "layer.h"

namespace lmoe {

constexpr int kG2K = 64;     // k-tile
constexpr int kXcds = 8;

template <int BM, int BN>
struct G2Shape {
    static constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    static constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 blocks per wave
    static constexpr int LA = BM * 8 / 256, LB = BN * 8 / 256;  // 16B loads per thread per k-tile
};

// 4 consecutive output columns of one row (c0 .. c0+3), epilogue per problem.
template <class E>
__device__ __forceinline__ void store_cols(E* dst, int c0, int ncols, const f32x4& v) {
    if (c0 + 3 < ncols && (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
        if constexpr (sizeof(E) == 2) {
            bf16 b[4] = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(b);
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
        for (int i = 0; i < 4; ++i)
            if (c0 + i < ncols) dst[i] = from_f32<E>(v[i]);
    }
}

template <class P>
struct RowCtx;  // per-row epilogue context, specialised per problem below

template <>
struct RowCtx<ProjRouter<bf16>> {
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4& v) {
        const int lz = a.standard ? 0 : a.l;
        if (c0 < lz) {
            store_cols(static_cast<bf16*>(a.z_w) + (size_t)r * a.l + c0, c0, lz, v);
        } else {
            const int e0 = c0 - lz;
            for (int i = 0; i < 4; ++i)
                if (e0 + i < a.N) a.logits[(size_t)r * a.N + e0 + i] = v[i] + (a.bias ? a.bias[e0 + i] : 0.0f);
        }
    }
};

template <>
struct RowCtx<Ffn1<bf16>> {
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4& v) {
        for (int i = 0; i < 4; ++i) {
            const float t = v[i] > 0.0f ? v[i] : 0.0f;
            v[i] = t * t;
        }
        store_cols(static_cast<bf16*>(a.abuf) + (size_t)slot * a.m + c0, c0, a.m, v);
    }
};

template <>
struct RowCtx<Ffn2<bf16, bf16>> {
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4& v) {
        const float g = a.gates[a.perm[slot]];
        for (int i = 0; i < 4; ++i) v[i] *= g;
        store_cols(static_cast<bf16*>(a.ybuf) + (size_t)slot * a.l + c0, c0, a.l, v);
    }
};

template <>
struct RowCtx<Up<bf16>> {
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4& v) {
        const bf16* xr = static_cast<const bf16*>(a.x) + (size_t)r * a.d + c0;
        if (c0 + 3 < a.d) {
            const uint2 u = *reinterpret_cast<const uint2*>(xr);
            v[0] += __uint_as_float(u.x << 16);
            v[1] += __uint_as_float(u.x & 0xffff0000u);
            v[2] += __uint_as_float(u.y << 16);
            v[3] += __uint_as_float(u.y & 0xffff0000u);
        } else {
            for (int i = 0; i < 4; ++i)
                if (c0 + i < a.d) v[i] += (float)xr[i];
        }
        store_cols(static_cast<bf16*>(a.out) + (size_t)r * a.d + c0, c0, a.d, v);
    }
};

template <class P, int BM, int BN>
__global__ __launch_bounds__(256) void gemm2_kernel(LayerArgs a, int nrow_tiles, int ncol_tiles) {
    using S = G2Shape<BM, BN>;
    // XCD-aware remap of the workgroup id to a logical tile; the grid is
    // kXcds * per_xcd workgroups, so every logical tile gets exactly one.
    const int G = nrow_tiles * ncol_tiles;
    const int per_xcd = (G + kXcds - 1) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= G) return;
    const int rt = logical / ncol_tiles, ct = logical % ncol_tiles;
    int grp, row0, row_end;
    if (!P::tile(a, rt, BM, grp, row0, row_end)) return;
    const int col0 = ct * BN;
    const int ncols = P::ncols(a);
    if (col0 >= ncols) return;
    const int K = P::kdim(a);
    const int nk = K / kG2K;

    __shared__ uint4 As[2][BM * 8];
    __shared__ uint4 Bs[2][BN * 8];

    const int tid = threadIdx.x;
    const int ch = tid & 7;   // 16-byte unit within a row's k-slice
    const int lrow = tid >> 3;
    // Rows past the tile's end (and columns past ncols) read a valid row
    // instead: each output element depends only on its own row and column,
    // and those outputs are never stored.  No load is conditional, so the
    // compiler can count the loads in flight exactly.
    const bf16* ap[S::LA];
    const bf16* bp[S::LB];
#pragma unroll
    for (int i = 0; i < S::LA; ++i) {
        const int r = row0 + lrow + 32 * i;
        ap[i] = P::a_row(a, grp, r < row_end ? r : row0) + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < S::LB; ++i) {
        const int c = col0 + lrow + 32 * i;
        bp[i] = P::b_row(a, grp, c < ncols ? c : col0) + ch * 8;
    }
    uint4 ra[S::LA], rb[S::LB];
    // Staged loads are split in 4 parts (load index i belongs to part i % 4),
    // so that part q of the next k-tile can go to LDS, and part q of the
    // k-tile after it can be loaded, right after MFMA group q.
    auto in_part = [](int i, int n, int q) { return n >= 4 ? (i % 4 == q) : (q == 0); };
    // the loads of a k-tile are issued during the first two MFMA groups, so
    // that they are at least two groups old when the next k-tile starts
    auto gload_group = [&](int kt, int g) {
        const int k0 = kt * kG2K;
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_part(i, S::LA, 2 * g) || in_part(i, S::LA, 2 * g + 1)) ra[i] = ldg16(ap[i] + k0);
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_part(i, S::LB, 2 * g) || in_part(i, S::LB, 2 * g + 1)) rb[i] = ldg16(bp[i] + k0);
    };
    auto swrite_part = [&](int st, int q) {
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_part(i, S::LA, q)) {
                const int r = lrow + 32 * i;
                As[st][r * 8 + (ch ^ (r & 7))] = ra[i];
            }
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_part(i, S::LB, q)) {
                const int r = lrow + 32 * i;
                Bs[st][r * 8 + (ch ^ (r & 7))] = rb[i];
            }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload_group(0, 0);
    gload_group(0, 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) swrite_part(0, q);
    __syncthreads();
    gload_group(min(1, nk - 1), 0);
    gload_group(min(1, nk - 1), 1);

    // Fragments of MFMA group kk+1 are read from LDS before the MFMAs of
    // group kk are issued (two register sets), so LDS latency overlaps them.
    auto read_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr) {
        const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
            const int r = wm * S::WM + i * 32 + (lane & 31);
            af[i] = as_bf16x8(As[st][r * 8 + (chunk ^ (r & 7))]);
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int c = wn * S::WN + j * 32 + (lane & 31);
            bfr[j] = as_bf16x8(Bs[st][c * 8 + (chunk ^ (c & 7))]);
        }
    };
    auto mfma_group = [&](const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    };
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        // the loop body is straight-line: the last iterations stage and load
        // a clamped k-tile that is never read
        const int kpre = min(kt + 2, nk - 1);
        bf16x8 a0[S::FM], b0[S::FN], a1[S::FM], b1[S::FN];
        read_frags(st, 0, a0, b0);
#pragma unroll
        for (int kk = 0; kk < kG2K / 16; ++kk) {
            bf16x8* ac = (kk & 1) ? a1 : a0;
            bf16x8* bc = (kk & 1) ? b1 : b0;
            bf16x8* an = (kk & 1) ? a0 : a1;
            bf16x8* bn = (kk & 1) ? b0 : b1;
            if (kk + 1 < kG2K / 16) read_frags(st, kk + 1, an, bn);
            if (kk < 2) {
                // parts 2kk, 2kk+1 of k-tile kt+1 go to LDS, then the same
                // registers take parts 2kk, 2kk+1 of k-tile kt+2
                swrite_part(st ^ 1, 2 * kk);
                swrite_part(st ^ 1, 2 * kk + 1);
                gload_group(kpre, kk);
            }
            mfma_group(ac, bc);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

    // epilogue: block (i, j), register group g: token row wm*WM + i*32 + lane%32,
    // columns wn*WN + j*32 + 8g + 4*(lane/32) + 0..3
#pragma unroll
    for (int i = 0; i < S::FM; ++i) {
        const int row = row0 + wm * S::WM + i * 32 + (lane & 31);
        if (row >= row_end) continue;
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = col0 + wn * S::WN + j * 32 + 8 * g + 4 * (lane >> 5);
                if (c < ncols) {
                    f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    RowCtx<P>::store(a, grp, row, c, v);
                }
            }
    }
}

}  // namespace lmoe
