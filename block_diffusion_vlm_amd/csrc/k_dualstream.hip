// Training-time dual-stream attention (Fast-dVLM overview §2.2.1-§2.2.2;
// Thai article §4.1, §4.4) over the vision-efficient token order
// [visual | clean text | noisy text]:
//   C2C  clean stream (visual + clean text) is token-level causal;
//   N2C  a noisy token sees every visual token and the clean text up to its
//        own position (the printed N2C matrix includes the diagonal);
//   N2N  noisy tokens attend bidirectionally inside their block;
//   no clean token sees a noisy one.
//
// bf16 path: flash attention forward on v_mfma_f32_32x32x16_bf16.  A
// workgroup owns 128 query rows of one head (4 waves x 32 rows) and streams
// 64-key tiles of K and V^T through LDS with an online softmax.  The mask is
// never materialised: for each query tile the visible key ranges follow in
// closed form from the three rules, every tile outside them is skipped, tiles
// that are visible for every (query, key) pair skip the per-element test,
// and only tiles crossing a rule boundary evaluate it.  Query tiles are
// launched heaviest first so that the long rows do not form a tail.
#include "attn_common.h"

namespace bd {

namespace {

using namespace attn;


// Headroom (log2 units) before the running maximum of a row is moved.
constexpr float kLazy = 8.0f;

struct Geometry {
    int n_vis, n_txt, ctx, N, block;
};

// Visibility of key j for query i (both < N).
__device__ __forceinline__ bool visible(const Geometry& G, int i, int j) {
    if (i < G.ctx) return j <= i;                      // C2C (j <= i < ctx)
    const int r = i - G.ctx;
    if (j < G.n_vis) return true;                      // N2C, visual keys
    if (j < G.ctx) return (j - G.n_vis) <= r;          // N2C, clean text
    return (j - G.ctx) / G.block == r / G.block;       // N2N
}

// Key ranges a query tile [i0, i1) must visit: range A = [0, a_end) (visual +
// clean keys), range B = [b_beg, b_end) (noisy keys, possibly empty).
__host__ __device__ inline void key_ranges(const Geometry& G, int i0, int i1, int* a_end,
                                           int* b_beg, int* b_end) {
    int ae = 0;
    if (i0 < G.ctx) ae = (i1 < G.ctx ? i1 : G.ctx);                 // clean rows: j <= i
    if (i1 > G.ctx) {
        const int r_last = i1 - 1 - G.ctx;
        const int noisy_reach = G.n_vis + r_last + 1;                // visual + clean <= r
        ae = ae > noisy_reach ? ae : noisy_reach;
        const int r_first = (i0 > G.ctx ? i0 : G.ctx) - G.ctx;
        *b_beg = G.ctx + (r_first / G.block) * G.block;
        int be = G.ctx + (r_last / G.block + 1) * G.block;
        *b_end = be < G.N ? be : G.N;
    } else {
        *b_beg = *b_end = 0;
    }
    *a_end = ae;
}

// True when every (query, key) pair of the tile is visible.
__device__ __forceinline__ bool tile_full(const Geometry& G, int i0, int i1, int j0, int j1) {
    if (i1 > G.N) i1 = G.N;
    if (j1 > G.N) return false;
    if (i1 <= G.ctx) return j1 - 1 <= i0;                            // causal, below diagonal
    if (i0 >= G.ctx) {
        const int r0 = i0 - G.ctx, r1 = i1 - 1 - G.ctx;
        if (j1 <= G.ctx) return j1 - 1 <= G.n_vis + r0;               // visual / clean text
        if (j0 >= G.ctx) {                                            // noisy keys
            const int b0 = r0 / G.block;
            return b0 == r1 / G.block && (j0 - G.ctx) / G.block == b0 &&
                   (j1 - 1 - G.ctx) / G.block == b0;
        }
    }
    return false;
}

// Visibility of keys for one query row as two intervals: key j is visible
// iff j <= lim or lo <= j < hi.  Clean row i: lim = i (C2C), no interval.
// Noisy row r: lim = n_vis + r (every visual key, clean text up to r: N2C),
// interval = the keys of its N2N block.
struct RowVis {
    int lim, lo, hi;
};

__device__ __forceinline__ RowVis row_vis(const Geometry& G, int i) {
    RowVis v;
    if (i < G.ctx) {
        v.lim = i;
        v.lo = v.hi = 0;
    } else {
        const int r = i - G.ctx;
        v.lim = G.n_vis + r;
        v.lo = G.ctx + (r / G.block) * G.block;
        v.hi = v.lo + G.block < G.N ? v.lo + G.block : G.N;
    }
    return v;
}

// WAVES waves per workgroup, each owning RB blocks of 32 query rows.  K/V
// tiles are double-buffered in LDS; the next tile's global loads are issued
// before the current tile is multiplied and land in the other buffer, so one
// barrier per tile suffices.
template <int WAVES, int RB, int OCC = 1>
__global__ __launch_bounds__(WAVES * 64, OCC) void dualstream_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Geometry G, int H, float scale_log2,
    uint16_t* __restrict__ out, int nqt) {
    constexpr int T = WAVES * 64;
    constexpr int BM = WAVES * 32 * RB;
    __shared__ __align__(16) Tiles tiles[2];
    const int h = blockIdx.x;
    // Later query tiles see more keys (causal context, then the visual prefix
    // plus clean text for the noisy stream), so tiles are issued last-first.
    const int qt = nqt - 1 - blockIdx.y;
    const int i0 = qt * BM;
    const int i1 = (i0 + BM < G.N) ? i0 + BM : G.N;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const size_t rs = size_t(H) * kDh;               // element stride between tokens

    int a_end, b_beg, b_end;
    key_ranges(G, i0, i1, &a_end, &b_beg, &b_end);
    const int na = (a_end + kBN - 1) / kBN;
    const int nb = b_end > b_beg ? (b_end - b_beg + kBN - 1) / kBN : 0;
    const int ntile = na + nb;
    const uint16_t* kb = k + size_t(h) * kDh;
    const uint16_t* vb = v + size_t(h) * kDh;
    auto tile_range = [&](int t, int& j0, int& jend) {
        if (t < na) {
            j0 = t * kBN;
            jend = a_end;
        } else {
            j0 = b_beg + (t - na) * kBN;
            jend = b_end;
        }
    };

    TileRegs<T> regs;
    if (ntile > 0) {
        int j0, jend;
        tile_range(0, j0, jend);
        fetch_tile<T>(regs, kb, vb, rs, j0, jend);
    }

    bf16x8 qf[RB][8];
    RowVis rv[RB];
    int rows[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = i0 + (wave * RB + rb) * 32 + (lane & 31);
        rows[rb] = row;
        const bool ok = row < G.N;
        load_q(qf[rb], ok ? q + size_t(row) * rs + size_t(h) * kDh : nullptr, lane);
        rv[rb] = ok ? row_vis(G, row) : RowVis{-1, 0, 0};
    }

    if (ntile > 0) store_tile<T>(tiles[0], regs);
    __syncthreads();

    float m[RB], l[RB];
    f32x16 oacc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m[rb] = -INFINITY;
        l[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[rb][db] = f32x16{};
    }

    for (int t = 0; t < ntile; ++t) {
        int j0, jend;
        tile_range(t, j0, jend);
        const int j1 = j0 + kBN < jend ? j0 + kBN : jend;
        if (t + 1 < ntile) {
            int n0, nend;
            tile_range(t + 1, n0, nend);
            fetch_tile<T>(regs, kb, vb, rs, n0, nend);
        }
        const Tiles& cur = tiles[t & 1];

        f32x16 sacc[RB][2];
        scores<RB>(sacc, cur, qf, lane);

        const bool full = (j1 - j0 == kBN) && tile_full(G, i0, i1, j0, j1);
        // Key of accumulator register e of this lane: jl + 8 (e / 4) + e % 4.
        const int jl = j0 + 4 * (lane >> 5);
        float x[RB][2][16];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (full) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int e = 0; e < 16; ++e) x[rb][kb2][e] = sacc[rb][kb2][e];
            } else {
                const int lim = rv[rb].lim < j1 - 1 ? rv[rb].lim : j1 - 1;
                const int hi = rv[rb].hi < j1 ? rv[rb].hi : j1;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = jl + 32 * kb2 + 8 * (e >> 2) + (e & 3);
                        const bool vis = (j <= lim) | ((j >= rv[rb].lo) & (j < hi));
                        x[rb][kb2][e] = vis ? sacc[rb][kb2][e] : -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, x[rb][kb2][e]);
            // Raw-score maximum, then everything in log2 units of the scaled
            // score.  The row's reference maximum m only moves when the new
            // maximum exceeds it by more than kLazy: until then probabilities
            // 2^(scale_log2 * s - m) stay below 2^kLazy, and skipping the
            // rescale of the running output leaves the final normalised
            // result unchanged.
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
            const bool move = mx > m[rb] + kLazy;
            const float mnew = move ? mx : m[rb];
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            float ls = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    x[rb][kb2][e] = __builtin_amdgcn_exp2f(fmaf(x[rb][kb2][e], scale_log2, -mref));
                    ls += x[rb][kb2][e];
                }
            ls += __shfl_xor(ls, 32);
            if (__ballot(move)) {
                const float alpha = __builtin_amdgcn_exp2f(m[rb] - mref);
                l[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[rb][db] *= alpha;
            }
            l[rb] += ls;
            m[rb] = mnew;
        }
        bf16x8 pf[RB][2][2];
        pack_p<RB>(pf, x);
        accumulate_pv<RB>(oacc, cur, pf, lane);

        if (t + 1 < ntile) store_tile<T>(tiles[(t + 1) & 1], regs);
        __syncthreads();
    }

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = rows[rb];
        if (row >= G.N) continue;
        const float inv = l[rb] > 0.f ? 1.f / l[rb] : 0.f;
        uint16_t* orow = out + size_t(row) * rs + size_t(h) * kDh;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int dh = 32 * db + acc_row(4 * e4, lane);
                bf16x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = static_cast<__bf16>(oacc[rb][db][4 * e4 + x] * inv);
                *reinterpret_cast<bf16x4*>(orow + dh) = w;
            }
    }
}

// float32 path: one wave per (token, head) row, online softmax over the
// visible keys in chunks of 64.
__global__ __launch_bounds__(64) void dualstream_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            Geometry G, int H, int dh,
                                                            float scale_log2,
                                                            float* __restrict__ out) {
    __shared__ float qs[128];
    const int i = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int lane = threadIdx.x;
    const size_t rs = size_t(H) * dh;
    for (int d = lane; d < dh; d += 64) qs[d] = q[size_t(i) * rs + size_t(h) * dh + d];
    __syncthreads();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 < G.N; j0 += 64) {
        const int j = j0 + lane;
        float x = -INFINITY;
        if (j < G.N && visible(G, i, j)) {
            const float* kr = k + size_t(j) * rs + size_t(h) * dh;
            float acc = 0.f;
            for (int d = 0; d < dh; ++d) acc = fmaf(qs[d], kr[d], acc);
            x = acc * scale_log2;
        }
        float cm = x;
        for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
        const float mn = fmaxf(m, cm);
        if (mn == -INFINITY) continue;
        const float alpha = exp2f(m - mn);
        const float p = exp2f(x - mn);
        float ps = p;
        for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
        l = l * alpha + ps;
        o0 *= alpha;
        o1 *= alpha;
        const int cnt = G.N - j0 < 64 ? G.N - j0 : 64;
        for (int t = 0; t < cnt; ++t) {
            const float pt = __shfl(p, t);
            const float* vr = v + size_t(j0 + t) * rs + size_t(h) * dh;
            if (lane < dh) o0 = fmaf(pt, vr[lane], o0);
            if (lane + 64 < dh) o1 = fmaf(pt, vr[lane + 64], o1);
        }
        m = mn;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = out + size_t(i) * rs + size_t(h) * dh;
    if (lane < dh) orow[lane] = o0 * inv;
    if (lane + 64 < dh) orow[lane + 64] = o1 * inv;
}

}  // namespace

#ifndef BD_DS_WAVES
#define BD_DS_WAVES 4
#endif
#ifndef BD_DS_RB
#define BD_DS_RB 1
#endif
#ifndef BD_DS_OCC
#define BD_DS_OCC 2
#endif

hipError_t launch_dualstream_bf16(const void* q, const void* k, const void* v, int n_vis,
                                  int n_txt, int block, int H, float scale, void* out,
                                  hipStream_t st) {
    constexpr int BM = BD_DS_WAVES * 32 * BD_DS_RB;
    Geometry G{n_vis, n_txt, n_vis + n_txt, n_vis + 2 * n_txt, block};
    const int nqt = (G.N + BM - 1) / BM;
    const dim3 grid(H, nqt);
    hipLaunchKernelGGL((dualstream_bf16_kernel<BD_DS_WAVES, BD_DS_RB, BD_DS_OCC>), grid,
                       dim3(BD_DS_WAVES * 64), 0, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), G, H,
                       scale * kLog2e, static_cast<uint16_t*>(out), nqt);
    return hipGetLastError();
}

hipError_t launch_dualstream_f32(const float* q, const float* k, const float* v, int n_vis,
                                 int n_txt, int block, int H, int dh, float scale, float* out,
                                 hipStream_t st) {
    Geometry G{n_vis, n_txt, n_vis + n_txt, n_vis + 2 * n_txt, block};
    hipLaunchKernelGGL(dualstream_f32_kernel, dim3(G.N * H), dim3(64), 0, st, q, k, v, G, H, dh,
                       scale * kLog2e, out);
    return hipGetLastError();
}

}  // namespace bd
