// Block attention at decode time: Bq block queries attend the KV-cached
// prefix (visual + prompt + earlier blocks, always visible) and the block's
// own keys under an intra-block bitmask (Fast-dVLM overview §1.2: blocks in
// order with a reusable KV cache, bidirectional denoising inside a block;
// §2.3.1 for the causal verify pass and the fused draft+verify mask).
//
// bf16 path: split-K over the keys (flash-decoding).  Grouped-query heads are
// packed so that all Bq x (Hq/Hkv) query rows of one KV head form the rows of
// one tile; workgroup (split, kv head, row block) handles 64 keys for up to
// 128 rows (4 waves x 32 rows) and writes a partial per row: its maximum and
// sum in float32 and its output normalised by that sum, O / l, in bfloat16
// (each value a convex combination of V rows, so bfloat16 keeps its range
// and costs the output at most about one more rounding of its own format);
// a second kernel merges the splits in a fixed order.
//
// FP8 KV cache (the fastest configuration of the overview runs FP8, §2.3.2):
// K and V hold OCP E4M3 codes with one float32 scale per KV head for each.
// Every E4M3 value is exact in bfloat16, so tiles are converted while they
// are staged into LDS and the bf16 MFMA path runs unchanged on the exact code
// values; the K scale joins the score scale and the V scale multiplies the
// partial outputs.
#include <type_traits>

#include "attn_common.h"

namespace bd {

namespace {

using namespace attn;

constexpr int kRowsPerWg = 128;

struct Partials {
    float* m;      // [rows][nsplit]
    float* l;      // [rows][nsplit]
    uint16_t* o;   // [rows][nsplit][128] bfloat16, O / l
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Partials partials(void* ws, int rows, int nsplit) {
    uint8_t* p = static_cast<uint8_t*>(ws);
    Partials r;
    r.m = reinterpret_cast<float*>(p);
    size_t off = al256(size_t(rows) * nsplit * 4);
    r.l = reinterpret_cast<float*>(p + off);
    off += al256(size_t(rows) * nsplit * 4);
    r.o = reinterpret_cast<uint16_t*>(p + off);
    return r;
}

inline size_t partials_bytes(int rows, int nsplit) {
    return 2 * al256(size_t(rows) * nsplit * 4) + al256(size_t(rows) * nsplit * kDh * 2);
}

// Paged cache: kc/vc are the page pools ([n_pages][Hkv][page_size][128]),
// key positions are logical, and the visited keys start at key_lo (prefix
// keys below it are left out); otherwise kc/vc are [Hkv][cap][128] and
// key_lo = 0.
struct Paging {
    const int32_t* table;
    int page_size, n_pages, key_lo;
};

// Per-KV-head scales of an FP8 cache (unused otherwise).
struct Fp8Kv {
    const float* k_scale;
    const float* v_scale;
};

// Eight E4M3 codes (two little-endian words) as bfloat16 values; exact.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), true);
    return bf16x8{static_cast<__bf16>(a[0]), static_cast<__bf16>(a[1]),
                  static_cast<__bf16>(b[0]), static_cast<__bf16>(b[1]),
                  static_cast<__bf16>(c[0]), static_cast<__bf16>(c[1]),
                  static_cast<__bf16>(d[0]), static_cast<__bf16>(d[1])};
}

// One 64-key tile of an FP8 cache in flight: thread t holds 32 codes (dh
// 32 (t % 4) .. +31) of key t / 4 of the tile, for K and for V.
struct Fp8Stage {
    u32x4 k[2], v[2];
};

template <bool PAGED, bool FP8 = false>
__global__ __launch_bounds__(256) void block_attn_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int P, const int32_t* __restrict__ P_dev, int cap,
    const uint64_t* __restrict__ mask, int Bq, int Hq, int Hkv, float scale_log2,
    void* __restrict__ ws, int nsplit, int kt, const int32_t* __restrict__ gate, Paging pg,
    Fp8Kv f8) {
    static_assert(!(PAGED && FP8), "the FP8 cache is contiguous");
    if (gated_off(gate)) return;
    // A device-side prefix length (the multi-block loop's kv_len) replaces P;
    // it never exceeds the host bound the grid and workspace were sized for.
    if (P_dev != nullptr) P = max(0, min(*P_dev, P));
    __shared__ __align__(16) uint16_t kbuf[2][kTile];
    __shared__ __align__(16) uint16_t vbuf[2][kTile];
    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int group = Hq / Hkv;
    const int R = Bq * group;                       // query rows of this KV head
    const int Nk = P + Bq;
    const uint16_t* kb = kc + size_t(g) * cap * kDh;
    const uint16_t* vb = vc + size_t(g) * cap * kDh;
    const int key_lo = PAGED ? pg.key_lo : 0;
    const int t_beg = split * kt;
    const int ntiles = (Nk - key_lo + kBN - 1) / kBN;
    if (t_beg >= ntiles) return;                    // past the keys of a shorter prefix
    const int t_end = t_beg + kt < ntiles ? t_beg + kt : ntiles;
    const unsigned koff = dma_lane_offset<false>(kDh);
    const unsigned voff = dma_lane_offset<true>(kDh);
    // FP8 cache: codes of tile t into registers (keys past the last one read
    // the last one), then converted into the swizzled bf16 LDS layouts.
    const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kc) + size_t(g) * cap * kDh;
    const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vc) + size_t(g) * cap * kDh;
    auto fetch8 = [&](int t, Fp8Stage& st) {
        const int j0 = t * kBN;
        const int n = Nk - j0 < kBN ? Nk - j0 : kBN;
        const int key = threadIdx.x >> 2;
        const size_t off = size_t(j0 + (key < n ? key : n - 1)) * kDh + 32 * (threadIdx.x & 3);
        st.k[0] = *reinterpret_cast<const u32x4*>(kb8 + off);
        st.k[1] = *reinterpret_cast<const u32x4*>(kb8 + off + 16);
        st.v[0] = *reinterpret_cast<const u32x4*>(vb8 + off);
        st.v[1] = *reinterpret_cast<const u32x4*>(vb8 + off + 16);
    };
    auto stage8 = [&](const Fp8Stage& st, uint16_t* kd, uint16_t* vd) {
        const int key = threadIdx.x >> 2;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int piece = 4 * (threadIdx.x & 3) + 2 * h2 + pp;   // 8 dh values
                *reinterpret_cast<bf16x8*>(kd + key * kDh + 8 * k_slot(key, piece)) =
                    e4m3x8_to_bf16(st.k[h2][2 * pp], st.k[h2][2 * pp + 1]);
                *reinterpret_cast<bf16x8*>(vd + key * kDh + 8 * v_slot(key, piece)) =
                    e4m3x8_to_bf16(st.v[h2][2 * pp], st.v[h2][2 * pp + 1]);
            }
    };
    auto load = [&](int t, uint16_t* kd, uint16_t* vd) {
        const int j0 = key_lo + t * kBN;
        const int n = Nk - j0 < kBN ? Nk - j0 : kBN;
        if constexpr (PAGED) {
            dma_tile_paged<4, false>(kd, kc, pg.table, pg.page_size, pg.n_pages, Hkv, g, j0, n);
            dma_tile_paged<4, true>(vd, vc, pg.table, pg.page_size, pg.n_pages, Hkv, g, j0, n);
        } else if (n == kBN) {
            dma_tile_full1<4, false>(lds_addr(kd), kb + size_t(j0) * kDh, kDh, koff);
            dma_tile_full1<4, true>(lds_addr(vd), vb + size_t(j0) * kDh, kDh, voff);
        } else {
            dma_tile<4, false>(kd, kb + size_t(j0) * kDh, kDh, n);
            dma_tile<4, true>(vd, vb + size_t(j0) * kDh, kDh, n);
        }
    };
    Fp8Stage st8;
    if constexpr (FP8) {
        fetch8(t_beg, st8);
        stage8(st8, kbuf[0], vbuf[0]);
    } else {
        load(t_beg, kbuf[0], vbuf[0]);
    }

    // Query row of this lane: r -> (block query i, head g*group + r % group).
    const int r = blockIdx.z * kRowsPerWg + wave * 32 + (lane & 31);
    const bool row_ok = r < R;
    const int qi = row_ok ? r / group : 0;
    const int qh = g * group + (row_ok ? r % group : 0);
    bf16x8 qf[8];
    load_q(qf, row_ok ? q + (size_t(qi) * Hq + qh) * kDh : nullptr, lane);
    // The row's intra-block mask; bits at or beyond Bq (keys past the block) are
    // never visible.
    const uint64_t mbits = row_ok ? mask[qi] & (Bq < 64 ? (1ull << Bq) - 1 : ~0ull) : 0;
    const ReadOffsets ro = read_offsets(lane);

    if constexpr (FP8) {
        // The query fragments are in before the loop: waited for at their
        // first use inside it, they would hold the MFMAs up behind the next
        // tile's code loads issued just before.
        dma_wait<0>();
        __syncthreads();
        scale_log2 *= f8.k_scale[g];
    } else {
        dma_wait<0>();
        tile_barrier();
    }

    float m = -INFINITY, l = 0.f;
    f32x16 oacc[4] = {};
    // One tile: the next tile's loads go into the other buffers (for an FP8
    // cache its codes are fetched here and staged after this tile).
    auto step = [&](int t, const uint16_t* kcur, const uint16_t* vcur, uint16_t* knxt,
                    uint16_t* vnxt) {
        const int j0 = key_lo + t * kBN;
        if constexpr (FP8) {
            if (t + 1 < t_end) fetch8(t + 1, st8);
        } else {
            if (t + 1 < t_end) load(t + 1, knxt, vnxt);
        }

        f32x16 sacc[2];
        scores(sacc, kcur, qf, ro);
        // Visibility of the lane's 32 score registers, one bit each.  Register
        // i (i / 16 = key block, i % 16 = e) holds the key at offset
        // 8 (i / 4) + i % 4 from the lane's first key jl.  Keys below P (the
        // prefix) form a prefix of the registers; a block key b = j - P is
        // visible by bit b of the row's mask, so the row's mask shifted to jl
        // has register i's bit at 8 (i / 4) + i % 4, and packing its low
        // nibbles gives the block part.
        const int jl = j0 + 4 * (lane >> 5);
        const int bb = jl - P;                      // block index of key jl
        uint64_t w = 0;
        if (bb >= 0) {
            if (bb < 64) w = mbits >> bb;
        } else if (bb > -64) {
            w = mbits << -bb;
        }
        w &= 0x0F0F0F0F0F0F0F0Full;
        w = (w | (w >> 4)) & 0x00FF00FF00FF00FFull;
        w = (w | (w >> 8)) & 0x0000FFFF0000FFFFull;
        w = (w | (w >> 16)) & 0x00000000FFFFFFFFull;
        const unsigned vis_bits = key_prefix(P - jl) | unsigned(w);
        float x[2][16];
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const unsigned sel = bit_select(vis_bits, 16 * kb2 + e);
                x[kb2][e] = __uint_as_float((__float_as_uint(sacc[kb2][e]) & sel) |
                                            (0xff800000u & ~sel));
                mx = fmaxf(mx, x[kb2][e]);
            }
        mx = fmaxf(mx, other_half(mx)) * scale_log2;
        const float mnew = fmaxf(m, mx);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        bf16x8 pf[2][2];
        float ls = exp_pack(pf, x, scale_log2, mref);
        ls += other_half(ls);
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        l = l * alpha + ls;
        m = mnew;
        // The first tile of a split finds oacc still zero: nothing to rescale.
        if (t != t_beg && __ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        }
        accumulate_pv(oacc, vcur, pf, ro);
        if constexpr (FP8) {
            if (t + 1 < t_end) stage8(st8, knxt, vnxt);
        }
    };
    // Loads (DMA) or staged stores (FP8) of the next tile complete before the
    // barrier; every wave has read the current tile after it.
    auto sync = [&] {
        if constexpr (FP8) {
            __syncthreads();
        } else {
            dma_wait<0>();
            tile_barrier();
        }
    };
    // One copy of the step in the code (the buffers alternate at run time):
    // short calls run one tile per split, on CUs whose instruction cache may
    // not hold this kernel, so its size shows in their latency.
    for (int t = t_beg; t < t_end; ++t) {
        const int cur = (t - t_beg) & 1;
        step(t, kbuf[cur], vbuf[cur], kbuf[cur ^ 1], vbuf[cur ^ 1]);
        sync();
    }
    if constexpr (FP8) {
        const float vs = f8.v_scale[g];
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= vs;
    }

    const Partials pt = partials(ws, Hkv * R, nsplit);
    if (row_ok && lane < 32) {
        const size_t rg = size_t(g) * R + r;        // global row
        pt.m[rg * nsplit + split] = m;
        pt.l[rg * nsplit + split] = l;
    }
    // The partial output leaves through LDS.  A lane holds pieces of its own
    // row only (four consecutive dims per accumulator group), so stores
    // straight from the accumulators would write 32 rows x 8 bytes per
    // instruction.  Each wave instead writes its 32 x 128 block of O / l, as
    // bfloat16, into one of the four tile buffers (free after the last
    // barrier of the loop), row-major: row rr holds sixteen 16-byte pieces
    // (8 dims each), piece c at slot c ^ (rr % 16), and a lane's four dims
    // fill one 8-byte half of a piece.  Read back as whole pieces, each
    // store instruction then writes four whole 256-byte rows.
    uint8_t* const region =
        reinterpret_cast<uint8_t*>(wave < 2 ? kbuf[wave] : vbuf[wave - 2]);
    const int rr = lane & 31;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            // dims 32 db + 8 e4 + 4 (lane / 32) .. + 3: piece 4 db + e4, half lane / 32
            const int c = 4 * db + e4;
            const bf16x4 w = {static_cast<__bf16>(oacc[db][4 * e4] * inv_l),
                              static_cast<__bf16>(oacc[db][4 * e4 + 1] * inv_l),
                              static_cast<__bf16>(oacc[db][4 * e4 + 2] * inv_l),
                              static_cast<__bf16>(oacc[db][4 * e4 + 3] * inv_l)};
            *reinterpret_cast<bf16x4*>(region + rr * 256 + 16 * (c ^ (rr & 15)) +
                                       8 * (lane >> 5)) = w;
        }
    const int r0 = blockIdx.z * kRowsPerWg + wave * 32;  // first query row of this wave
    const int c = lane & 15;
    u32x4 val[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = 4 * it + (lane >> 4);
        val[it] = *reinterpret_cast<const u32x4*>(region + row * 256 + 16 * (c ^ (row & 15)));
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = 4 * it + (lane >> 4);
        if (r0 + row < R) {
            const size_t rg = size_t(g) * R + r0 + row;
            *reinterpret_cast<u32x4*>(pt.o + (rg * nsplit + split) * kDh + 8 * c) = val[it];
        }
    }
}

// One workgroup of 128 threads per query row; thread t owns output dim t.
// The splits are taken kCombineBatch at a time and every load of a batch is
// issued before any is used, so a batch costs one memory round trip: lane u
// of each wave reads split s0 + u's maximum and sum (vector loads), every
// thread reads its output dim of each split, and the weights 2^(m_s - M) are
// broadcast from their lanes with readlane.  Splits are accumulated in a
// fixed order; the running maximum moves once per batch.
constexpr int kCombineThreads = 128;
constexpr int kCombineBatch = 32;

__global__ __launch_bounds__(kCombineThreads) void block_attn_combine_kernel(
    const void* __restrict__ ws, int Bq, int Hq, int Hkv, int nsplit, uint16_t* __restrict__ out,
    const int32_t* __restrict__ gate, int P, const int32_t* __restrict__ P_dev, int kt) {
    if (gated_off(gate)) return;
    // With a device-side prefix length only the splits that hold keys were
    // written; nsplit stays the row stride of the partials.
    int nsplit_used = nsplit;
    if (P_dev != nullptr) {
        const int Pd = max(0, min(*P_dev, P));
        nsplit_used = ((Pd + Bq + kBN - 1) / kBN + kt - 1) / kt;
    }
    const int rg = blockIdx.x;                      // global row = g * R + r
    const int group = Hq / Hkv;
    const int R = Bq * group;
    const int g = rg / R;
    const int r = rg % R;
    const int qi = r / group;
    const int qh = g * group + r % group;
    const int t = threadIdx.x;
    const int u_lane = t & (kCombineBatch - 1);
    const Partials pt = partials(const_cast<void*>(ws), Hkv * R, nsplit);
    const float* m = pt.m + size_t(rg) * nsplit;
    const float* l = pt.l + size_t(rg) * nsplit;
    const uint16_t* o = pt.o + size_t(rg) * nsplit * kDh + t;

    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < nsplit_used; s0 += kCombineBatch) {
        // Past the last split the last one is read again and dropped.
        const int su = min(s0 + u_lane, nsplit_used - 1);
        float mu = m[su];
        const float lu = l[su];
        float ov[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            ov[u] = bf16_to_f32(o[size_t(min(s0 + u, nsplit_used - 1)) * kDh]);
        if (s0 + u_lane >= nsplit_used) mu = -INFINITY;
        float mb = mu;                              // batch maximum (lanes 32..63 mirror 0..31)
        for (int off = kCombineBatch / 2; off > 0; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
        // No branch here, so that the output loads stay next to the others.
        const float Mn = fmaxf(M, mb);
        const float a = (Mn == -INFINITY) ? 1.f : exp2f(M - Mn);  // 0 while M is -inf
        const float wu = (mu == -INFINITY) ? 0.f : exp2f(mu - Mn);
        L *= a;
        acc *= a;
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wu), u));
            const float lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lu), u));
            const float wl = w * lw;                // split weight of its O / l
            L += wl;
            acc += wl * ov[u];
        }
        M = Mn;
    }
    const float res = (M == -INFINITY) ? 0.f : acc / L;
    const float nb = __shfl_down(res, 1);
    if ((t & 1) == 0) {
        uint16_t* dst = out + (size_t(qi) * Hq + qh) * kDh + t;
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(res, nb);
    }
}

// ---------------------------------------------------------------------------
// float32 path: one wave per (query, head) row, keys in chunks of 64 with an
// online softmax; lanes own keys for the scores and dims for the output.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void block_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    int P, int cap, const uint64_t* __restrict__ mask, int Bq, int Hq, int Hkv, int dh,
    float scale_log2, float* __restrict__ out, const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    __shared__ float qs[128];
    const int qi = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int g = h / (Hq / Hkv);
    const int lane = threadIdx.x;
    const float* qr = q + (size_t(qi) * Hq + h) * dh;
    for (int d = lane; d < dh; d += 64) qs[d] = qr[d];
    __syncthreads();
    const uint64_t mbits = mask[qi];
    const float* kb = kc + size_t(g) * cap * dh;
    const float* vb = vc + size_t(g) * cap * dh;
    const int Nk = P + Bq;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 < Nk; j0 += 64) {
        const int j = j0 + lane;
        float x = -INFINITY;
        if (j < Nk && (j < P || ((mbits >> (j - P)) & 1ull))) {
            const float* kr = kb + size_t(j) * dh;
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
        const int cnt = Nk - j0 < 64 ? Nk - j0 : 64;
        for (int t = 0; t < cnt; ++t) {
            const float pt = __shfl(p, t);
            const float* vr = vb + size_t(j0 + t) * dh;
            if (lane < dh) o0 = fmaf(pt, vr[lane], o0);
            if (lane + 64 < dh) o1 = fmaf(pt, vr[lane + 64], o1);
        }
        m = mn;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = out + (size_t(qi) * Hq + h) * dh;
    if (lane < dh) orow[lane] = o0 * inv;
    if (lane + 64 < dh) orow[lane + 64] = o1 * inv;
}

// Key tiles per workgroup.  A decode-sized call is bound by latency: each
// split runs a chain of dependent steps per tile, so the fewest tiles per
// split win while the grid (splits x KV heads x 128-row blocks) is small;
// every split also writes a partial row per query row, which the merge
// reads back.  A split takes the fewest tiles that keep the grid within half
// the chip (one workgroup per CU) as long as that is at most
// kMaxTilesHalf tiles, and otherwise the fewest that keep it within the
// whole chip, which also bounds the partial outputs when the prefix is long.
// (Measured against the whole-chip rule alone: 0.65 us less at 2 x 16
// queries over 4,608 keys (3 tiles per split instead of 2) and at 16 over
// 20,016 (5 instead of 3); 16 tiles instead of 8 at 65,536 keys took 8 us
// more, hence the bound.)
constexpr int kSplitCUs = 256;                       // compute units of the chip
constexpr int kMaxTilesHalf = 6;

int workgroups_per_split(int Bq, int Hq, int Hkv) {
    const int R = Bq * (Hq / Hkv);
    return Hkv * ((R + kRowsPerWg - 1) / kRowsPerWg);
}

int max_splits(int Bq, int Hq, int Hkv) {
    const int m = kSplitCUs / workgroups_per_split(Bq, Hq, Hkv);
    return m > 1 ? m : 1;
}

int tiles_per_split(int P, int Bq, int Hq, int Hkv) {
    const int ntiles = (P + Bq + kBN - 1) / kBN;
    const int mh = kSplitCUs / 2 / workgroups_per_split(Bq, Hq, Hkv);
    if (mh >= 1) {
        const int kt = ntiles > mh ? (ntiles + mh - 1) / mh : 1;
        if (kt <= kMaxTilesHalf) return kt;
    }
    const int m = max_splits(Bq, Hq, Hkv);
    return ntiles > m ? (ntiles + m - 1) / m : 1;
}

int num_splits(int P, int Bq, int Hq, int Hkv) {
    const int ntiles = (P + Bq + kBN - 1) / kBN;
    const int kt = tiles_per_split(P, Bq, Hq, Hkv);
    return (ntiles + kt - 1) / kt;
}

hipError_t launch_block_attn_any(const void* q, const void* kc, const void* vc, int P, int cap,
                                 const uint64_t* mask, int Bq, int Hq, int Hkv, float scale,
                                 void* out, void* ws, hipStream_t st, const int32_t* gate,
                                 Paging pg, const Fp8Kv* f8 = nullptr,
                                 const int32_t* P_dev = nullptr) {
    // Splits over the visited keys [key_lo, P + Bq).
    const int kt = tiles_per_split(P - pg.key_lo, Bq, Hq, Hkv);
    const int nsplit = num_splits(P - pg.key_lo, Bq, Hq, Hkv);
    const int R = Bq * (Hq / Hkv);
    const dim3 grid(nsplit, Hkv, (R + kRowsPerWg - 1) / kRowsPerWg);
    if (f8 != nullptr)
        hipLaunchKernelGGL((block_attn_split_kernel<false, true>), grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                           static_cast<const uint16_t*>(vc), P, P_dev, cap, mask, Bq, Hq, Hkv,
                           scale * kLog2e, ws, nsplit, kt, gate, pg, *f8);
    else if (pg.table != nullptr)
        hipLaunchKernelGGL(block_attn_split_kernel<true>, grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                           static_cast<const uint16_t*>(vc), P, P_dev, cap, mask, Bq, Hq, Hkv,
                           scale * kLog2e, ws, nsplit, kt, gate, pg, Fp8Kv{});
    else
        hipLaunchKernelGGL(block_attn_split_kernel<false>, grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                           static_cast<const uint16_t*>(vc), P, P_dev, cap, mask, Bq, Hq, Hkv,
                           scale * kLog2e, ws, nsplit, kt, gate, pg, Fp8Kv{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(block_attn_combine_kernel, dim3(Bq * Hq), dim3(kCombineThreads), 0, st, ws,
                       Bq, Hq, Hkv, nsplit, static_cast<uint16_t*>(out), gate, P, P_dev, kt);
    return hipGetLastError();
}

}  // namespace

// Sized for min(ntiles, max_splits) splits, an upper bound of num_splits
// that never decreases with P, so a workspace sized for one prefix length
// serves every shorter one (the multi-block loop sizes it for its last
// block).
size_t block_attn_ws_bytes(int P, int Bq, int Hq, int Hkv, int dh) {
    (void)dh;
    const int ntiles = (P + Bq + kBN - 1) / kBN;
    const int m = max_splits(Bq, Hq, Hkv);
    return partials_bytes(Bq * Hq, ntiles < m ? ntiles : m);
}

hipError_t launch_block_attn_bf16(const void* q, const void* kc, const void* vc, int P, int cap,
                                  const uint64_t* mask, int Bq, int Hq, int Hkv, float scale,
                                  void* out, void* ws, hipStream_t st, const int32_t* gate,
                                  const int32_t* P_dev) {
    return launch_block_attn_any(q, kc, vc, P, cap, mask, Bq, Hq, Hkv, scale, out, ws, st, gate,
                                 Paging{nullptr, 1, 1, 0}, nullptr, P_dev);
}

hipError_t launch_block_attn_fp8kv(const void* q, const uint8_t* kc, const uint8_t* vc,
                                   const float* k_scale, const float* v_scale, int P, int cap,
                                   const uint64_t* mask, int Bq, int Hq, int Hkv, float scale,
                                   void* out, void* ws, hipStream_t st) {
    const Fp8Kv f8{k_scale, v_scale};
    return launch_block_attn_any(q, kc, vc, P, cap, mask, Bq, Hq, Hkv, scale, out, ws, st, nullptr,
                                 Paging{nullptr, 1, 1, 0}, &f8);
}

// New K or V rows into an FP8 cache: row i of head g goes to cache row pos + i.
// Four elements per thread: fl32(x * fl32(1 / scale)), clamped to +-448,
// rounded to E4M3 (nearest, ties to even).
__global__ __launch_bounds__(256) void kv_quant_fp8_kernel(const uint16_t* __restrict__ x, int n,
                                                           int Hkv, int dh,
                                                           const float* __restrict__ scale,
                                                           uint8_t* __restrict__ cache, int cap,
                                                           int pos) {
    const size_t i4 = (size_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
    const size_t total = size_t(n) * Hkv * dh;
    if (i4 >= total) return;
    const int d = int(i4 % dh);
    const size_t rh = i4 / dh;                       // row * Hkv + head
    const int g = int(rh % Hkv);
    const int row = int(rh / Hkv);
    const float inv = 1.0f / scale[g];
    const uint2 w = *reinterpret_cast<const uint2*>(x + i4);
    float f[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = fminf(fmaxf(f[e] * inv, -448.f), 448.f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
    *reinterpret_cast<int*>(cache + (size_t(g) * cap + pos + row) * dh + d) = packed;
}

hipError_t launch_kv_quant_fp8(const void* x, int n, int Hkv, int dh, const float* scale,
                               uint8_t* cache, int cap, int pos, hipStream_t st) {
    const size_t quads = size_t(n) * Hkv * dh / 4;
    if (quads == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_quant_fp8_kernel, dim3(unsigned((quads + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), n, Hkv, dh, scale, cache, cap, pos);
    return hipGetLastError();
}

hipError_t launch_block_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* page_table, int page_size, int n_pages, int P,
                                   int key_lo, const uint64_t* mask, int Bq, int Hq, int Hkv,
                                   float scale, void* out, void* ws, hipStream_t st) {
    return launch_block_attn_any(q, k_pool, v_pool, P, 0, mask, Bq, Hq, Hkv, scale, out, ws, st,
                                 nullptr, Paging{page_table, page_size, n_pages, key_lo});
}


hipError_t launch_block_attn_f32(const float* q, const float* kc, const float* vc, int P, int cap,
                                 const uint64_t* mask, int Bq, int Hq, int Hkv, int dh,
                                 float scale, float* out, hipStream_t st, const int32_t* gate) {
    hipLaunchKernelGGL(block_attn_f32_kernel, dim3(Bq * Hq), dim3(64), 0, st, q, kc, vc, P, cap,
                       mask, Bq, Hq, Hkv, dh, scale * kLog2e, out, gate);
    return hipGetLastError();
}

}  // namespace bd
