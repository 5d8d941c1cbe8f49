// Training-time dual-stream attention (Fast-dVLM overview §2.2.1-§2.2.2;
// Thai article §4.1, §4.4) over the vision-efficient token order
// [visual | clean text | noisy text]:
//   C2C  clean stream (visual + clean text) is token-level causal;
//   N2C  a noisy token sees every visual token and the clean text up to its
//        own position (the printed N2C matrix includes the diagonal);
//   N2N  noisy tokens attend bidirectionally inside their block;
//   no clean token sees a noisy one.
// With the auto-truncation mask (overview §2.2.2; Thai article §4.3) the text
// is split into segments (the turns' prompts and responses): N2N blocks tile
// every segment from its own start and end at the segment's end, so the last
// block of a response never reaches into the next prompt.  One segment is
// the plain mask.
//
// bf16 path: flash attention forward on v_mfma_f32_32x32x16_bf16.  A
// workgroup owns 128 query rows of one head (4 waves x 32 rows), two
// workgroups share a CU, and 64-key tiles of K and V stream through LDS with
// an online softmax.  The mask is never materialised: for each query tile the
// visible key ranges follow in closed form from the three rules, every tile
// outside them is skipped, tiles that are visible for every (query, key) pair
// skip the per-element test, and only tiles crossing a rule boundary
// evaluate it.  Query tiles are launched heaviest first so that the long
// rows do not form a tail.
#include <type_traits>

#include "attn_common.h"
#include "dualstream_common.h"

namespace bd {

namespace {

using namespace attn;
using namespace ds;


// Headroom (log2 units) before the running maximum of a row is moved.
constexpr float kLazy = 8.0f;

// One wave per 32 query rows, WAVES waves per workgroup sharing the K/V
// tiles, two waves per SIMD.  The scores of tile t+1 are computed while the
// softmax of tile t runs: the score block of an iteration is laid out as 16
// issue slots separated by scheduling barriers, each issuing one K fragment
// read (two slots ahead of its use), one score MFMA and a share of the
// softmax's vector work, so that the vector ALUs work while the MFMAs
// execute; the P V MFMAs of tile t follow, with their V fragment reads issued
// two slots ahead.  K runs one tile ahead of V: iteration t reads K(t+1) and
// V(t) and loads K(t+2) and V(t+1) into the other halves of two double
// buffers (complete tiles with per-lane offsets computed once); one barrier
// per iteration separates the loads from their readers.
template <int WAVES, bool SEG, bool LSE>
__global__ __launch_bounds__(WAVES * 64, 2) void dualstream_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Geometry G, int H, float scale_log2,
    uint16_t* __restrict__ out, int nqt, float* __restrict__ lse) {
    constexpr int BM = WAVES * 32;
    constexpr int kAhead = 2;                        // fragment reads issued ahead
    __shared__ __align__(16) uint16_t kbuf[2][kTile];
    __shared__ __align__(16) uint16_t vbuf[2][kTile];
    const int h = blockIdx.x;
    // Later query tiles see more keys (causal context, then the visual prefix
    // plus clean text for the noisy stream), so tiles are issued last-first.
    const int qt = nqt - 1 - blockIdx.y;
    const int i0 = qt * BM;
    const int i1 = (i0 + BM < G.N) ? i0 + BM : G.N;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rs = H * kDh;                          // element stride between tokens

    int a_end, b_beg, b_end;
    key_ranges<SEG>(G, i0, i1, &a_end, &b_beg, &b_end);
    const int na = (a_end + kBN - 1) / kBN;
    const int nb = b_end > b_beg ? (b_end - b_beg + kBN - 1) / kBN : 0;
    const int ntile = na + nb;
    // A complete tile of range A is visible for every (query, key) pair of a
    // wave when its last key is at most full_a: below the causal diagonal
    // for clean rows, inside visual + clean text up to the first row for
    // noisy rows, taken from the wave's first row (the choice is per wave:
    // nothing inside a tile step synchronises the waves).
    // A complete tile of range B is when all rows lie in one noisy block
    // (range B is then exactly that block's keys).
    const int iw0 = i0 + 32 * (threadIdx.x >> 6);    // the wave's first row
    const int full_a = i1 <= G.ctx ? iw0 : (i0 >= G.ctx ? G.n_vis + (iw0 - G.ctx) : -1);
    bool full_b = false;
    if (i0 >= G.ctx) {
        int lo0, hi0, lo1, hi1;
        noisy_block<SEG>(G, i0 - G.ctx, &lo0, &hi0);
        noisy_block<SEG>(G, i1 - 1 - G.ctx, &lo1, &hi1);
        full_b = lo0 == lo1;
    }
    const uint16_t* kh = k + size_t(h) * kDh;
    const uint16_t* vh = v + size_t(h) * kDh;
    auto tile_j0 = [&](int t) { return t < na ? t * kBN : b_beg + (t - na) * kBN; };
    auto tile_n = [&](int t) {
        const int n = (t < na ? a_end : b_end) - tile_j0(t);
        return n < kBN ? n : kBN;
    };
    const unsigned koff = dma_lane_offset<false>(rs);
    const unsigned voff = dma_lane_offset<true>(rs);
    // Tiles past the last one are replaced by the last one (their buffers are
    // not read).  Destinations are LDS byte addresses of buffer halves.
    const unsigned kbuf_lds = lds_addr(&kbuf[0][0]);
    const unsigned vbuf_lds = lds_addr(&vbuf[0][0]);
    auto load_k = [&](int t, int half) {
        const unsigned dst = kbuf_lds + unsigned(half) * (2u * kTile);
        t = t < ntile ? t : ntile - 1;
        const int n = tile_n(t);
        if (n == kBN)
            dma_tile_full1<WAVES, false>(dst, kh + size_t(tile_j0(t)) * rs, rs, koff);
        else
            dma_tile<WAVES, false>(dst, kh + size_t(tile_j0(t)) * rs, rs, n);
    };
    auto load_v = [&](int t, int half) {
        const unsigned dst = vbuf_lds + unsigned(half) * (2u * kTile);
        t = t < ntile ? t : ntile - 1;
        const int n = tile_n(t);
        if (n == kBN)
            dma_tile_full1<WAVES, true>(dst, vh + size_t(tile_j0(t)) * rs, rs, voff);
        else
            dma_tile<WAVES, true>(dst, vh + size_t(tile_j0(t)) * rs, rs, n);
    };
    if (ntile <= 0) return;                          // every row sees at least key 0

    load_k(0, 0);
    load_k(1, 1);
    load_v(0, 0);
    const ReadOffsets ro = read_offsets(lane);
    const int row = i0 + wave * 32 + (lane & 31);
    const bool row_ok = row < G.N;
    bf16x8 qf[8];
    load_q(qf, row_ok ? q + size_t(row) * rs + size_t(h) * kDh : nullptr, lane);
    const RowVis rv = row_ok ? row_vis<SEG>(G, row) : RowVis{-1, 0, 0};
    float m = -INFINITY, l = 0.f;
    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    dma_wait<0>();
    tile_barrier();
    f32x16 sA[2], sB[2];
    scores(sA, kbuf[0], qf, ro);
    tile_barrier();           // every wave has read K(0) before K(2) replaces it

    // Score block of iteration t: S(t+1) from kread into snext, with the
    // softmax of tile t (scores s) into the bf16 P^T fragments p.  MASKED
    // evaluates the visibility rules per element (tiles not visible as a
    // whole).  Slots [0, kMax) take the row maximum, slot kMax decides the
    // reference maximum, the remaining slots exponentiate pairs of elements,
    // pack them to bf16 and add them to the row sum (four partial maxima and
    // sums keep the reduction chains short).  A row's reference maximum m only
    // moves when the new maximum exceeds it by more than kLazy (log2 units of
    // the scaled score): until then probabilities stay below 2^kLazy, and
    // skipping the rescale of the running output leaves the final normalised
    // result unchanged.
    auto score_block = [&](auto masked_tag, int j0, int j1, const f32x16 (&s)[2],
                           f32x16 (&snext)[2], const uint16_t* kread, bf16x8 (&p)[2][2],
                           float& mnew, float& mref, float& ls, bool& move) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr int kMax = MASKED ? 4 : 2;
        constexpr int kExp = 16 - kMax - 1;
        auto rk = [&](int i) { return read_k(kread, ro, i & 1, i >> 1); };
        bf16x8 ka[16];
        static_for<0, kAhead>([&](auto I) { ka[I] = rk(I); });
        // Visible registers of a partly visible tile, one bit each: keys up
        // to lim, and keys in [lo, hi), both cut at the tile's end j1.
        unsigned vis_bits = 0xffffffffu;
        if constexpr (MASKED) {
            const int jl = j0 + 4 * (lane >> 5);        // this lane's first key
            const int lim = rv.lim < j1 - 1 ? rv.lim : j1 - 1;
            const int hi = rv.hi < j1 ? rv.hi : j1;
            vis_bits = key_prefix(lim - jl + 1) |
                       (key_prefix(hi - jl) & ~key_prefix(rv.lo - jl));
        }
        auto val = [&](int e) -> float {
            if constexpr (MASKED) {
                const unsigned sel = bit_select(vis_bits, e);
                return __uint_as_float((__float_as_uint(s[e >> 4][e & 15]) & sel) |
                                       (0xff800000u & ~sel));
            } else {
                return s[e >> 4][e & 15];
            }
        };
        float mxp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        float lsp[4] = {0.f, 0.f, 0.f, 0.f};
        const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        static_for<0, 16>([&](auto Ic) {
            constexpr int i = Ic;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (i + kAhead < 16) ka[i + kAhead] = rk(i + kAhead);
            // key blocks alternate, so consecutive MFMAs are independent
            snext[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                ka[i], qf[i >> 1], i < 2 ? f32x16{} : snext[i & 1], 0, 0, 0);
            if constexpr (i < kMax) {
                constexpr int per = 32 / kMax;
                static_for<i * per, (i + 1) * per>(
                    [&](auto Ec) { mxp[int(Ec) & 3] = fmaxf(mxp[int(Ec) & 3], val(Ec)); });
            } else if constexpr (i == kMax) {
                float mx = fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
                mx = fmaxf(mx, other_half(mx)) * scale_log2;
                move = mx > m + kLazy;
                mnew = move ? mx : m;
                mref = (mnew == -INFINITY) ? 0.f : mnew;
            } else {
                constexpr int q0 = i - kMax - 1;
                constexpr int p_beg = (q0 * 16) / kExp;
                constexpr int p_end = ((q0 + 1) * 16) / kExp;
                float pe[32];
                static_for<2 * p_beg, 2 * p_end>([&](auto Ec) {
                    pe[int(Ec)] = __builtin_amdgcn_exp2f(fmaf(val(Ec), scale_log2, -mref));
                });
                static_for<p_beg, p_end>([&](auto Pc) {
                    constexpr int e = 2 * int(Pc);
                    const bf16x2 two = {static_cast<__bf16>(pe[e]),
                                        static_cast<__bf16>(pe[e + 1])};
                    constexpr int kb = e >> 4, s2 = (e & 15) >> 3, eo = e & 7;
                    p[kb][s2][eo] = two[0];
                    p[kb][s2][eo + 1] = two[1];
                    lsp[int(Pc) & 3] =
                        __builtin_amdgcn_fdot2_f32_bf16(two, one, lsp[int(Pc) & 3], false);
                });
                if constexpr (i == 15) {
                    ls = (lsp[0] + lsp[1]) + (lsp[2] + lsp[3]);
                    ls += other_half(ls);
                }
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    // P V of one tile from vread: 16 issue slots, one V fragment read (two
    // slots ahead of its use) and one MFMA each; dh blocks alternate.
    auto pv_block = [&](const uint16_t* vread, const bf16x8 (&p)[2][2]) {
        auto rvv = [&](int j) { return read_v(vread, ro, j & 3, j >> 3, (j >> 2) & 1); };
        bf16x8 va[16];
        static_for<0, kAhead>([&](auto J) { va[J] = rvv(J); });
        static_for<0, 16>([&](auto Jc) {
            constexpr int j = Jc;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (j + kAhead < 16) va[j + kAhead] = rvv(j + kAhead);
            oacc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], p[j >> 3][(j >> 2) & 1],
                                                                  oacc[j & 3], 0, 0, 0);
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    // Iteration t: reads K(t+1) and V(t); loads K(t+2) where K(t) was and
    // V(t+1) where V(t-1) was.
    auto step = [&](int t, const f32x16 (&s)[2], f32x16 (&snext)[2]) {
        load_k(t + 2, t & 1);
        load_v(t + 1, (t + 1) & 1);
        const int j0 = tile_j0(t);
        const int n = tile_n(t);
        const bool full = n == kBN && (t < na ? j0 + kBN - 1 <= full_a : full_b);
        bf16x8 p[2][2];
        float mnew, mref, ls;
        bool move;
        if (full)
            score_block(std::false_type{}, j0, j0 + n, s, snext, kbuf[(t + 1) & 1], p, mnew,
                        mref, ls, move);
        else
            score_block(std::true_type{}, j0, j0 + n, s, snext, kbuf[(t + 1) & 1], p, mnew,
                        mref, ls, move);
        // Rescale what tiles 0 .. t-1 accumulated when the reference maximum
        // of a row moved (alpha is 1 for the others).
        if (__ballot(move)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mref);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        }
        l += ls;
        m = mnew;
        pv_block(vbuf[t & 1], p);
    };
    int t = 0;
    for (;;) {
        step(t, sA, sB);
        dma_wait<0>();
        tile_barrier();
        if (++t == ntile) break;
        step(t, sB, sA);
        dma_wait<0>();
        tile_barrier();
        if (++t == ntile) break;
    }

    if (!row_ok) return;
    // Row log-sum-exp (natural log) for the backward: the sum of
    // 2^(x scale_log2) over the visible keys is 2^m l.
    if (LSE && lane < 32)
        lse[size_t(row) * H + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = out + size_t(row) * rs + size_t(h) * kDh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d = 32 * db + acc_row(4 * e4, lane);
            bf16x4 w;
#pragma unroll
            for (int x = 0; x < 4; ++x) w[x] = static_cast<__bf16>(oacc[db][4 * e4 + x] * inv);
            *reinterpret_cast<bf16x4*>(orow + d) = w;
        }
}

// float32 path: one wave per (token, head) row, online softmax over the
// visible keys in chunks of 64.
__global__ __launch_bounds__(64) void dualstream_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            Geometry G, int H, int dh,
                                                            float scale_log2,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
    __shared__ float qs[128];
    const int i = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int lane = threadIdx.x;
    const size_t rs = size_t(H) * dh;
    for (int d = lane; d < dh; d += 64) qs[d] = q[size_t(i) * rs + size_t(h) * dh + d];
    __syncthreads();
    const RowVis rv = row_vis<true>(G, i);
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 < G.N; j0 += 64) {
        const int j = j0 + lane;
        float x = -INFINITY;
        if (j < G.N && (j <= rv.lim || (j >= rv.lo && j < rv.hi))) {
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
    if (lse != nullptr && lane == 0)
        lse[size_t(i) * H + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = out + size_t(i) * rs + size_t(h) * dh;
    if (lane < dh) orow[lane] = o0 * inv;
    if (lane + 64 < dh) orow[lane + 64] = o1 * inv;
}

}  // namespace

hipError_t launch_dualstream_bf16(const void* q, const void* k, const void* v, int n_vis,
                                  int n_txt, int block, int H, float scale, void* out,
                                  hipStream_t st, const int32_t* seg, int n_seg, float* lse) {
    constexpr int kWaves = 4;
    constexpr int BM = kWaves * 32;
    const Geometry G = make_geometry(n_vis, n_txt, block, seg, n_seg);
    const int nqt = (G.N + BM - 1) / BM;
    const dim3 grid(H, nqt);
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    auto* oo = static_cast<uint16_t*>(out);
    const float sl = scale * kLog2e;
    const dim3 blk(kWaves * 64);
    if (G.n_seg > 1) {
        if (lse)
            hipLaunchKernelGGL((dualstream_bf16_kernel<kWaves, true, true>), grid, blk, 0, st, qq,
                               kk, vv, G, H, sl, oo, nqt, lse);
        else
            hipLaunchKernelGGL((dualstream_bf16_kernel<kWaves, true, false>), grid, blk, 0, st,
                               qq, kk, vv, G, H, sl, oo, nqt, lse);
    } else {
        if (lse)
            hipLaunchKernelGGL((dualstream_bf16_kernel<kWaves, false, true>), grid, blk, 0, st,
                               qq, kk, vv, G, H, sl, oo, nqt, lse);
        else
            hipLaunchKernelGGL((dualstream_bf16_kernel<kWaves, false, false>), grid, blk, 0, st,
                               qq, kk, vv, G, H, sl, oo, nqt, lse);
    }
    return hipGetLastError();
}

hipError_t launch_dualstream_f32(const float* q, const float* k, const float* v, int n_vis,
                                 int n_txt, int block, int H, int dh, float scale, float* out,
                                 hipStream_t st, const int32_t* seg, int n_seg, float* lse) {
    const Geometry G = make_geometry(n_vis, n_txt, block, seg, n_seg);
    hipLaunchKernelGGL(dualstream_f32_kernel, dim3(G.N * H), dim3(64), 0, st, q, k, v, G, H, dh,
                       scale * kLog2e, out, lse);
    return hipGetLastError();
}

}  // namespace bd
