// Training backward of the dual-stream attention (Fast-dVLM overview
// §2.2.1-§2.2.2; Thai article §4.1, §4.3): the gradients of masked softmax
// attention under the N2N / N2C / C2C masks (with the auto-truncation
// segments, when given),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale dS K,  dK = scale dS^T Q,
// with P = exp(scale Q K^T - lse) recomputed from the row log-sum-exp that
// the forward kept, so no N x N matrix is ever stored.
//
// bf16 path, on v_mfma_f32_32x32x16_bf16 with the forward's building blocks:
//   1. D per (row, head) from O and dO (a small float32 kernel);
//   2. dQ: a workgroup owns 128 query rows (4 waves x 32) and visits the key
//      tiles the rows see, exactly as the forward does; per tile
//      S^T = K Q^T and dP^T = V dO^T (both with the tile as the A operand),
//      dS^T in registers, dQ^T += K^T dS^T (K^T by transposing LDS reads);
//   3. dK and dV: a workgroup owns 128 keys (4 waves x 32, the keys' K and V
//      rows held as B operands) and visits the query-row tiles that see them;
//      per tile S = Q K^T and dP = dO V^T (the row tile as the A operand),
//      P and dS in registers, dV^T += dO^T P and dK^T += Q^T dS.
// Each kernel writes every output element once; nothing is accumulated with
// atomics, so the result is deterministic.  Row and key tiles come from the
// closed-form visibility rules; the per-element test runs on every tile.
#include <type_traits>

#include "attn_common.h"
#include "dualstream_common.h"

namespace bd {

namespace {

using namespace attn;
using namespace ds;

constexpr int kRowsPerWg = 128;      // 4 waves x 32 rows (dQ) or keys (dK, dV)
// Operand reads issued this many MFMAs ahead of their use: the dK/dV kernel
// runs one wave per SIMD, so its reads cannot hide behind another wave.
constexpr int kAheadDq = 2;
constexpr int kAheadDkdv = 4;

__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// D[r] = sum_d dO[r][d] O[r][d] for every (token, head) row r = token * H +
// head: 16 lanes per row (float32 path; the bf16 dQ kernel forms D itself).
template <typename T>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const T* __restrict__ out,
                                                         const T* __restrict__ dout, int rows,
                                                         int dh, float* __restrict__ D) {
    const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    float acc = 0.f;
    if (r < rows) {
        const T* o = out + size_t(r) * dh;
        const T* g = dout + size_t(r) * dh;
        for (int d = l; d < dh; d += 16) acc = fmaf(to_f32(o[d]), to_f32(g[d]), acc);
    }
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (l == 0 && r < rows) D[r] = acc;
}

// Stores a wave's transposed 32 x 128 result (accumulator layout, lane =
// row or key, registers = dh) as one bf16 row of `dst`, times `mul`.
__device__ __forceinline__ void store_rowT(uint16_t* dst, const f32x16 (&acc)[4], float mul,
                                           int lane) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d = 32 * db + acc_row(4 * e4, lane);
            bf16x4 w;
#pragma unroll
            for (int x = 0; x < 4; ++x) w[x] = static_cast<__bf16>(acc[db][4 * e4 + x] * mul);
            *reinterpret_cast<bf16x4*>(dst + d) = w;
        }
}

// ---------------------------------------------------------------------------
// dQ: 128 query rows per workgroup, key tiles of 64.  Each workgroup first
// forms D = rowsum(dO * O) of its rows from the dO fragments it holds anyway
// and writes it, with the rows' log-sum-exp in log2 units, for the dK/dV
// kernel that runs after it.
// ---------------------------------------------------------------------------
template <bool SEG>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ out, const float* __restrict__ lse, float* __restrict__ D,
    float* __restrict__ lse2_out, Geometry G, int H, float scale_log2, float scale,
    uint16_t* __restrict__ dq, int nqt) {
    __shared__ __align__(16) uint16_t kK[kTile];     // K tile, A-operand layout
    __shared__ __align__(16) uint16_t kV[kTile];     // K tile, transposed-read layout
    __shared__ __align__(16) uint16_t vK[kTile];     // V tile, A-operand layout
    const int h = blockIdx.x;
    const int qt = nqt - 1 - blockIdx.y;             // longest rows first
    const int i0 = qt * kRowsPerWg;
    const int i1 = (i0 + kRowsPerWg < G.N) ? i0 + kRowsPerWg : G.N;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rs = H * kDh;

    int a_end, b_beg, b_end;
    key_ranges<SEG>(G, i0, i1, &a_end, &b_beg, &b_end);
    const int na = (a_end + kBN - 1) / kBN;
    const int nb = b_end > b_beg ? (b_end - b_beg + kBN - 1) / kBN : 0;
    const int ntile = na + nb;
    auto tile_j0 = [&](int t) { return t < na ? t * kBN : b_beg + (t - na) * kBN; };
    auto tile_n = [&](int t) {
        const int n = (t < na ? a_end : b_end) - tile_j0(t);
        return n < kBN ? n : kBN;
    };

    const int row = i0 + wave * 32 + (lane & 31);
    const bool row_ok = row < G.N;
    bf16x8 qf[8], gf[8];
    load_q(qf, row_ok ? q + size_t(row) * rs + size_t(h) * kDh : nullptr, lane);
    load_q(gf, row_ok ? dout + size_t(row) * rs + size_t(h) * kDh : nullptr, lane);
    const float lse2 = row_ok ? lse[size_t(row) * H + h] * kLog2e : INFINITY;
    // D of this lane's row: lanes l and l + 32 hold complementary halves of
    // dO (load_q's layout), so each adds its half and takes the other's.
    float Dr;
    {
        bf16x8 of[8];
        load_q(of, row_ok ? out + size_t(row) * rs + size_t(h) * kDh : nullptr, lane);
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = fmaf(static_cast<float>(of[s][e]), static_cast<float>(gf[s][e]), acc);
        Dr = acc + other_half(acc);
    }
    if (row_ok && lane < 32) {
        D[size_t(row) * H + h] = Dr;
        lse2_out[size_t(row) * H + h] = lse2;
    }
    const RowVis rv = row_ok ? row_vis<SEG>(G, row) : RowVis{-1, 0, 0};
    const ReadOffsets ro = read_offsets(lane);
    const uint16_t* kh = k + size_t(h) * kDh;
    const uint16_t* vh = v + size_t(h) * kDh;

    f32x16 dqacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dqacc[db] = f32x16{};
    for (int t = 0; t < ntile; ++t) {
        const int j0 = tile_j0(t);
        const int n = tile_n(t);
        dma_tile<4, false>(kK, kh + size_t(j0) * rs, rs, n);
        dma_tile<4, true>(kV, kh + size_t(j0) * rs, rs, n);
        dma_tile<4, false>(vK, vh + size_t(j0) * rs, rs, n);
        dma_wait<0>();
        tile_barrier();
        f32x16 sacc[2], dpacc[2];
        scores_ahead<kAheadDq>(sacc, kK, qf, ro);    // S^T[key][row]
        scores_ahead<kAheadDq>(dpacc, vK, gf, ro);   // dP^T[key][row] = V[key] . dO[row]
        bf16x8 dsf[2][2];
        auto grad = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            // Visible keys of this lane's registers (bit e for register e):
            // keys up to lim or in [lo, hi), and inside the tile.
            unsigned vis_bits = 0xffffffffu;
            if constexpr (MASKED) {
                const int jl = j0 + 4 * (lane >> 5);
                vis_bits = key_prefix(n - 4 * (lane >> 5)) &
                           (key_prefix(rv.lim - jl + 1) |
                            (key_prefix(rv.hi - jl) & ~key_prefix(rv.lo - jl)));
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], scale_log2, -lse2));
                    if constexpr (MASKED)
                        p = __uint_as_float(__float_as_uint(p) & bit_select(vis_bits, 16 * kb + e));
                    dsf[kb][e >> 3][e & 7] = static_cast<__bf16>(p * (dpacc[kb][e] - Dr));
                }
        };
        // A tile that every row of the wave sees whole skips the selection
        // (rows past the end take no part: their results are dropped).  The
        // segmented instance always selects: a second copy of the step would
        // not fit its registers.
        const bool whole = n == kBN && (!row_ok || rv.lim >= j0 + kBN - 1 ||
                                        (rv.lo <= j0 && rv.hi >= j0 + kBN));
        if (!SEG && __all(whole))
            grad(std::false_type{});
        else
            grad(std::true_type{});
        accumulate_pv_ahead<kAheadDq>(dqacc, kV, dsf, ro);   // dQ^T += K^T dS^T
        tile_barrier();                              // the tile is read before it is replaced
    }
    if (!row_ok) return;
    store_rowT(dq + size_t(row) * rs + size_t(h) * kDh, dqacc, scale, lane);
}

// ---------------------------------------------------------------------------
// dK, dV: 128 keys per workgroup, query-row tiles of 64, two tiles in LDS:
// the loads of tile t+1 (Q and dO in both layouts, and the rows' lse and D)
// run while tile t is multiplied.
// ---------------------------------------------------------------------------
template <bool SEG>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ D, Geometry G, int H,
    float scale_log2, float scale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    // [buffer][Q A-operand, Q transposed-read, dO A-operand, dO transposed-read]
    __shared__ __align__(16) uint16_t tiles[2][4][kTile];
    __shared__ __align__(16) float lse_s[2][kBN];
    __shared__ __align__(16) float D_s[2][kBN];
    const int h = blockIdx.x;
    const int j0w = blockIdx.y * kRowsPerWg;         // keys seen by the most rows first
    const int j1w = (j0w + kRowsPerWg < G.N) ? j0w + kRowsPerWg : G.N;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rs = H * kDh;

    int a_beg, b_beg, b_end;
    row_ranges<SEG>(G, j0w, j1w, &a_beg, &b_beg, &b_end);
    const int na = a_beg < G.ctx ? (G.ctx - a_beg + kBN - 1) / kBN : 0;
    const int nb = b_end > b_beg ? (b_end - b_beg + kBN - 1) / kBN : 0;
    const int ntile = na + nb;
    auto tile_i0 = [&](int t) { return t < na ? a_beg + t * kBN : b_beg + (t - na) * kBN; };
    auto tile_n = [&](int t) {
        const int n = (t < na ? G.ctx : b_end) - tile_i0(t);
        return n < kBN ? n : kBN;
    };

    const int key = j0w + wave * 32 + (lane & 31);
    const bool key_ok = key < G.N;
    bf16x8 kf[8], vf[8];
    load_q(kf, key_ok ? k + size_t(key) * rs + size_t(h) * kDh : nullptr, lane);
    load_q(vf, key_ok ? v + size_t(key) * rs + size_t(h) * kDh : nullptr, lane);
    // The fragments are consumed here, so that the compiler completes their
    // loads before the tile loop: a wait for them inside the loop would also
    // wait for the next tile's loads, which it does not track.
#pragma unroll
    for (int s = 0; s < 8; ++s) __asm__ volatile("" ::"v"(kf[s]), "v"(vf[s]));
    // An absent key (past N) is seen by no row.
    const KeyVis kv = key_ok ? key_vis<SEG>(G, key) : KeyVis{G.N, G.n_txt, 0, 0};
    const ReadOffsets ro = read_offsets(lane);
    const uint16_t* qh = q + size_t(h) * kDh;
    const uint16_t* gh = dout + size_t(h) * kDh;

    // Loads of row tile t into buffer b: 16 per wave, plus the 64 rows' lse
    // and D (wave 0, two more).
    auto issue = [&](int t, int b) {
        const int i0 = tile_i0(t);
        const int n = tile_n(t);
        dma_tile<4, false>(tiles[b][0], qh + size_t(i0) * rs, rs, n);
        dma_tile<4, true>(tiles[b][1], qh + size_t(i0) * rs, rs, n);
        dma_tile<4, false>(tiles[b][2], gh + size_t(i0) * rs, rs, n);
        dma_tile<4, true>(tiles[b][3], gh + size_t(i0) * rs, rs, n);
        if (wave == 0) {
            dma_floats64(lse_s[b], lse2 + h, H, i0, i0 + n - 1);
            dma_floats64(D_s[b], D + h, H, i0, i0 + n - 1);
        }
    };

    // A row tile is visible from every key of a complete key range when its
    // rows are clean and all at or after the last key, or noisy and the keys
    // all visual or clean text at or before the first row's position; such
    // tiles skip the per-element test.
    const bool keys_full = j1w - j0w == kRowsPerWg;
    auto tile_full = [&](int i0, int n) {
        if (!keys_full || n != kBN) return false;
        if (i0 + n <= G.ctx) return j1w - 1 <= i0;
        if (i0 >= G.ctx) return j1w <= G.ctx && (i0 - G.ctx) >= (j1w - 1 - G.n_vis);
        return false;
    };

    f32x16 dkacc[4], dvacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }
    if (ntile > 0) issue(0, 0);
    for (int t = 0; t < ntile; ++t) {
        const int b = t & 1;
        if (t + 1 < ntile) {
            issue(t + 1, b ^ 1);
            // this tile's loads have landed; the next tile's stay in flight
            if (wave == 0)
                dma_wait<18>();
            else
                dma_wait<16>();
        } else {
            dma_wait<0>();
        }
        tile_barrier();
        const int i0 = tile_i0(t);
        const int n = tile_n(t);
        f32x16 sacc[2], dpacc[2];
        scores_ahead<kAheadDkdv>(sacc, tiles[b][0], kf, ro);    // S[row][key]
        scores_ahead<kAheadDkdv>(dpacc, tiles[b][2], vf, ro);   // dP[row][key] = dO[row] . V[key]
        bf16x8 pf[2][2], dsf[2][2];
        const int il = 4 * (lane >> 5);
        auto grad = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            // Rows of this lane's registers that see the key (bit e for
            // register e; rows at offsets from i0 + il): clean rows at or
            // after the key; noisy rows from rmin on or inside [lo, hi);
            // all inside the tile.  A tile is all clean or all noisy.
            unsigned vis_bits = 0xffffffffu;
            if constexpr (MASKED) {
                const int base = i0 + il;
                if (i0 < G.ctx) {
                    vis_bits = ~key_prefix(kv.j - base);
                } else {
                    const int rb = base - G.ctx;
                    vis_bits = ~key_prefix(kv.rmin - rb) |
                               (key_prefix(kv.hi - rb) & ~key_prefix(kv.lo - rb));
                }
                vis_bits &= key_prefix(n - il);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int ir0 = 32 * kb + il + 8 * e4;   // rows ir0 .. ir0 + 3 of the tile
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[b][ir0]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&D_s[b][ir0]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int e = 4 * e4 + x;
                        float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], scale_log2, -l4[x]));
                        if constexpr (MASKED)
                            p = __uint_as_float(__float_as_uint(p) &
                                                bit_select(vis_bits, 16 * kb + e));
                        pf[kb][e >> 3][e & 7] = static_cast<__bf16>(p);
                        dsf[kb][e >> 3][e & 7] =
                            static_cast<__bf16>(p * (dpacc[kb][e] - d4[x]));
                    }
                }
        };
        if (tile_full(i0, n))
            grad(std::false_type{});
        else
            grad(std::true_type{});
        accumulate_pv_ahead<kAheadDkdv>(dvacc, tiles[b][3], pf, ro);    // dV^T += dO^T P
        accumulate_pv_ahead<kAheadDkdv>(dkacc, tiles[b][1], dsf, ro);   // dK^T += Q^T dS
        tile_barrier();                              // buffer b is read before it is refilled
    }
    if (!key_ok) return;
    store_rowT(dk + size_t(key) * rs + size_t(h) * kDh, dkacc, scale, lane);
    store_rowT(dv + size_t(key) * rs + size_t(h) * kDh, dvacc, 1.f, lane);
}

// ---------------------------------------------------------------------------
// float32 path (small problems): one wave per (row, head) for dQ and one per
// (key, head) for dK, dV; lanes own keys (rows) for the scores and head
// dimensions for the outputs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    Geometry G, int H, int dh, float scale, float* __restrict__ dq) {
    __shared__ float qs[128], gs[128];
    const int i = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int lane = threadIdx.x;
    const size_t rs = size_t(H) * dh;
    for (int d = lane; d < dh; d += 64) {
        qs[d] = q[size_t(i) * rs + size_t(h) * dh + d];
        gs[d] = dout[size_t(i) * rs + size_t(h) * dh + d];
    }
    __syncthreads();
    const RowVis rv = row_vis<true>(G, i);
    const float li = lse[size_t(i) * H + h];
    const float Di = D[size_t(i) * H + h];
    float a0 = 0.f, a1 = 0.f;
    for (int j0 = 0; j0 < G.N; j0 += 64) {
        const int j = j0 + lane;
        float ds = 0.f;
        if (j < G.N && (j <= rv.lim || (j >= rv.lo && j < rv.hi))) {
            const float* kr = k + size_t(j) * rs + size_t(h) * dh;
            const float* vr = v + size_t(j) * rs + size_t(h) * dh;
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < dh; ++d) {
                s = fmaf(qs[d], kr[d], s);
                dp = fmaf(gs[d], vr[d], dp);
            }
            const float p = exp2f((s * scale - li) * kLog2e);
            ds = p * (dp - Di);
        }
        const int cnt = G.N - j0 < 64 ? G.N - j0 : 64;
        for (int t = 0; t < cnt; ++t) {
            const float dst = __shfl(ds, t);
            const float* kr = k + size_t(j0 + t) * rs + size_t(h) * dh;
            if (lane < dh) a0 = fmaf(dst, kr[lane], a0);
            if (lane + 64 < dh) a1 = fmaf(dst, kr[lane + 64], a1);
        }
    }
    float* o = dq + size_t(i) * rs + size_t(h) * dh;
    if (lane < dh) o[lane] = a0 * scale;
    if (lane + 64 < dh) o[lane + 64] = a1 * scale;
}

__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ D,
    Geometry G, int H, int dh, float scale, float* __restrict__ dk, float* __restrict__ dv) {
    __shared__ float ks[128], vs[128];
    const int j = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int lane = threadIdx.x;
    const size_t rs = size_t(H) * dh;
    for (int d = lane; d < dh; d += 64) {
        ks[d] = k[size_t(j) * rs + size_t(h) * dh + d];
        vs[d] = v[size_t(j) * rs + size_t(h) * dh + d];
    }
    __syncthreads();
    const KeyVis kv = key_vis<true>(G, j);
    float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
    for (int i0 = 0; i0 < G.N; i0 += 64) {
        const int i = i0 + lane;
        float p = 0.f, ds = 0.f;
        if (i < G.N && seen_by(G, kv, i)) {
            const float* qr = q + size_t(i) * rs + size_t(h) * dh;
            const float* gr = dout + size_t(i) * rs + size_t(h) * dh;
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < dh; ++d) {
                s = fmaf(qr[d], ks[d], s);
                dp = fmaf(gr[d], vs[d], dp);
            }
            p = exp2f((s * scale - lse[size_t(i) * H + h]) * kLog2e);
            ds = p * (dp - D[size_t(i) * H + h]);
        }
        const int cnt = G.N - i0 < 64 ? G.N - i0 : 64;
        for (int t = 0; t < cnt; ++t) {
            const float pt = __shfl(p, t);
            const float dst = __shfl(ds, t);
            const float* qr = q + size_t(i0 + t) * rs + size_t(h) * dh;
            const float* gr = dout + size_t(i0 + t) * rs + size_t(h) * dh;
            if (lane < dh) {
                v0 = fmaf(pt, gr[lane], v0);
                k0 = fmaf(dst, qr[lane], k0);
            }
            if (lane + 64 < dh) {
                v1 = fmaf(pt, gr[lane + 64], v1);
                k1 = fmaf(dst, qr[lane + 64], k1);
            }
        }
    }
    float* ko = dk + size_t(j) * rs + size_t(h) * dh;
    float* vo = dv + size_t(j) * rs + size_t(h) * dh;
    if (lane < dh) {
        ko[lane] = k0 * scale;
        vo[lane] = v0;
    }
    if (lane + 64 < dh) {
        ko[lane + 64] = k1 * scale;
        vo[lane + 64] = v1;
    }
}

template <typename T>
hipError_t launch_rowdot(const T* out, const T* dout, int rows, int dh, float* D,
                         hipStream_t st) {
    hipLaunchKernelGGL(bwd_rowdot_kernel<T>, dim3((rows + 15) / 16), dim3(256), 0, st, out, dout,
                       rows, dh, D);
    return hipGetLastError();
}

}  // namespace

// D, then (bf16 path) the row log-sum-exp in log2 units, [N][H] float32 each.
size_t dualstream_bwd_ws_bytes(int N, int H) {
    return 2 * (((size_t(N) * H * sizeof(float)) + 255) & ~size_t(255));
}

hipError_t launch_dualstream_bwd_bf16(const void* q, const void* k, const void* v,
                                      const void* out, const void* dout, const float* lse,
                                      int n_vis, int n_txt, int block, const int32_t* seg,
                                      int n_seg, int H, float scale, void* dq, void* dk, void* dv,
                                      void* ws, hipStream_t st) {
    const Geometry G = make_geometry(n_vis, n_txt, block, seg, n_seg);
    float* D = static_cast<float*>(ws);
    float* lse2 = D + dualstream_bwd_ws_bytes(G.N, H) / 2 / sizeof(float);
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    const auto* gg = static_cast<const uint16_t*>(dout);
    const auto* oo = static_cast<const uint16_t*>(out);
    const int nt = (G.N + kRowsPerWg - 1) / kRowsPerWg;
    const dim3 grid(H, nt), blk(256);
    const float sl = scale * kLog2e;
    if (G.n_seg > 1) {
        hipLaunchKernelGGL(bwd_dq_kernel<true>, grid, blk, 0, st, qq, kk, vv, gg, oo, lse, D, lse2,
                           G, H, sl, scale, static_cast<uint16_t*>(dq), nt);
        hipLaunchKernelGGL(bwd_dkdv_kernel<true>, grid, blk, 0, st, qq, kk, vv, gg, lse2, D, G, H,
                           sl, scale, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
    } else {
        hipLaunchKernelGGL(bwd_dq_kernel<false>, grid, blk, 0, st, qq, kk, vv, gg, oo, lse, D,
                           lse2, G, H, sl, scale, static_cast<uint16_t*>(dq), nt);
        hipLaunchKernelGGL(bwd_dkdv_kernel<false>, grid, blk, 0, st, qq, kk, vv, gg, lse2, D, G, H,
                           sl, scale, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
    }
    return hipGetLastError();
}

hipError_t launch_dualstream_bwd_f32(const float* q, const float* k, const float* v,
                                     const float* out, const float* dout, const float* lse,
                                     int n_vis, int n_txt, int block, const int32_t* seg,
                                     int n_seg, int H, int dh, float scale, float* dq, float* dk,
                                     float* dv, void* ws, hipStream_t st) {
    const Geometry G = make_geometry(n_vis, n_txt, block, seg, n_seg);
    float* D = static_cast<float*>(ws);
    hipError_t e = launch_rowdot(out, dout, G.N * H, dh, D, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3(G.N * H), dim3(64), 0, st, q, k, v, dout, lse, D,
                       G, H, dh, scale, dq);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3(G.N * H), dim3(64), 0, st, q, k, v, dout, lse,
                       D, G, H, dh, scale, dk, dv);
    return hipGetLastError();
}

}  // namespace bd
