// Geometry of the dual-stream token order [visual | clean text | noisy
// text] and the closed-form visibility rules shared by the forward and
// backward kernels (Fast-dVLM overview §2.2.1-§2.2.2; Thai article §4.1,
// §4.3):
//   C2C  the clean stream (visual + clean text) is token-level causal;
//   N2C  a noisy token sees every visual token and the clean text up to its
//        own position;
//   N2N  noisy tokens see each other inside their block; blocks tile every
//        text segment from its start and end at its end (auto-truncation);
//   no clean token sees a noisy one.
#pragma once

#include "bd_internal.h"

namespace bd {
namespace ds {

struct Geometry {
    int n_vis, n_txt, ctx, N, block;
    int n_seg;                          // text segments, 1 .. kMaxSegments
    int seg[kMaxSegments];              // their starts (text positions), seg[0] = 0
};

// The N2N block [lo, hi) (text positions) of noisy text position r: blocks
// tile r's segment from its start and are cut at its end.  SEG = false is
// the one-segment case.  The scan has static indices only, so the segment
// starts stay in kernel-argument (scalar) memory.
template <bool SEG = true>
__host__ __device__ inline void noisy_block(const Geometry& G, int r, int* lo, int* hi) {
    if constexpr (!SEG) {
        *lo = (r / G.block) * G.block;
        *hi = *lo + G.block < G.n_txt ? *lo + G.block : G.n_txt;
        return;
    }
    int s0 = 0, s1 = G.n_txt;
#pragma unroll
    for (int s = 1; s < kMaxSegments; ++s) {
        if (s < G.n_seg) {
            const int b = G.seg[s];
            if (b <= r)
                s0 = b;
            else if (b < s1)
                s1 = b;
        }
    }
    *lo = s0 + ((r - s0) / G.block) * G.block;
    *hi = *lo + G.block < s1 ? *lo + G.block : s1;
}

// Key ranges a query tile [i0, i1) must visit: range A = [0, a_end) (visual +
// clean keys), range B = [b_beg, b_end) (noisy keys, possibly empty).
template <bool SEG>
__host__ __device__ inline void key_ranges(const Geometry& G, int i0, int i1, int* a_end,
                                           int* b_beg, int* b_end) {
    int ae = 0;
    if (i0 < G.ctx) ae = (i1 < G.ctx ? i1 : G.ctx);                 // clean rows: j <= i
    if (i1 > G.ctx) {
        const int r_last = i1 - 1 - G.ctx;
        const int noisy_reach = G.n_vis + r_last + 1;                // visual + clean <= r
        ae = ae > noisy_reach ? ae : noisy_reach;
        const int r_first = (i0 > G.ctx ? i0 : G.ctx) - G.ctx;
        int lo, hi;
        noisy_block<SEG>(G, r_first, &lo, &hi);
        *b_beg = G.ctx + lo;
        noisy_block<SEG>(G, r_last, &lo, &hi);
        *b_end = G.ctx + hi;
    } else {
        *b_beg = *b_end = 0;
    }
    *a_end = ae;
}

// Visibility of keys for one query row as two intervals: key j is visible
// iff j <= lim or lo <= j < hi.  Clean row i: lim = i (C2C), no interval.
// Noisy row r: lim = n_vis + r (every visual key, clean text up to r: N2C),
// interval = the keys of its N2N block.
struct RowVis {
    int lim, lo, hi;
};

template <bool SEG>
__device__ __forceinline__ RowVis row_vis(const Geometry& G, int i) {
    RowVis v;
    if (i < G.ctx) {
        v.lim = i;
        v.lo = v.hi = 0;
    } else {
        const int r = i - G.ctx;
        v.lim = G.n_vis + r;
        int lo, hi;
        noisy_block<SEG>(G, r, &lo, &hi);
        v.lo = G.ctx + lo;
        v.hi = G.ctx + hi;
    }
    return v;
}

// Visibility of one key j from the query side, for the backward pass: row i
// sees key j iff (i < ctx and j <= i) or (i >= ctx and, with r = i - ctx,
// r >= rmin or lo <= r < hi).  Visual key: rmin = 0; clean text key at text
// position t: rmin = t; noisy key at text position t: no rmin (n_txt), and
// [lo, hi) = t's N2N block.
struct KeyVis {
    int j, rmin, lo, hi;
};

template <bool SEG>
__device__ __forceinline__ KeyVis key_vis(const Geometry& G, int j) {
    KeyVis v{j, G.n_txt, 0, 0};
    if (j < G.n_vis) {
        v.rmin = 0;
    } else if (j < G.ctx) {
        v.rmin = j - G.n_vis;
    } else {
        noisy_block<SEG>(G, j - G.ctx, &v.lo, &v.hi);
    }
    return v;
}

__device__ __forceinline__ bool seen_by(const Geometry& G, const KeyVis& kv, int i) {
    if (i < G.ctx) return kv.j <= i;
    const int r = i - G.ctx;
    return (r >= kv.rmin) | ((r >= kv.lo) & (r < kv.hi));
}

// Query rows a key tile [j0, j1) is seen from: clean rows [a_beg, ctx) and
// noisy rows [b_beg, b_end) (either possibly empty; the noisy range is the
// hull of the clean keys' rows and the noisy keys' blocks).
template <bool SEG>
__host__ __device__ inline void row_ranges(const Geometry& G, int j0, int j1, int* a_beg,
                                           int* b_beg, int* b_end) {
    *a_beg = j0 < G.ctx ? j0 : G.ctx;
    int bb = G.N, be = G.ctx;
    if (j0 < G.n_vis) {
        bb = G.ctx;
        be = G.N;
    } else if (j0 < G.ctx) {
        bb = G.ctx + (j0 - G.n_vis);
        be = G.N;
    }
    if (j1 > G.ctx) {
        int lo, hi, lo2, hi2;
        noisy_block<SEG>(G, (j0 > G.ctx ? j0 : G.ctx) - G.ctx, &lo, &hi);
        noisy_block<SEG>(G, j1 - 1 - G.ctx, &lo2, &hi2);
        const int nb = G.ctx + lo, ne = G.ctx + hi2;
        if (bb >= be) {
            bb = nb;
            be = ne;
        } else {
            bb = bb < nb ? bb : nb;
            be = be > ne ? be : ne;
        }
    }
    *b_beg = bb;
    *b_end = be;
}

// Host: the geometry of a call; seg (n_seg entries) holds the segment starts,
// null for one segment.
inline Geometry make_geometry(int n_vis, int n_txt, int block, const int32_t* seg, int n_seg) {
    Geometry G{};
    G.n_vis = n_vis;
    G.n_txt = n_txt;
    G.ctx = n_vis + n_txt;
    G.N = n_vis + 2 * n_txt;
    G.block = block;
    G.n_seg = seg != nullptr ? n_seg : 1;
    for (int s = 0; s < G.n_seg; ++s) G.seg[s] = seg != nullptr ? seg[s] : 0;
    return G;
}

}  // namespace ds
}  // namespace bd
