// Pieces shared by the LM-head kernels (bf16 and FP8): the layout of the
// per-workgroup partial states in the workspace, the fold of four logits into
// a running (max, sum, argmax) state, the end-of-kernel reduction of a
// workgroup's states, and the choice of the persistent grid.
#pragma once

#include "bd_internal.h"

namespace bd {

constexpr int kMaxGrid = 256;       // persistent workgroups of the streaming kernels

// Partial states live column-major, [position][partial], so that the merge
// kernel reads each position's partials with coalesced loads.
struct WsView {
    float* m;
    float* s;
    int* a;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline WsView ws_view(void* ws, int G, int B) {
    uint8_t* p = static_cast<uint8_t*>(ws);
    const size_t one = align256(size_t(G) * B * sizeof(float));
    WsView v;
    v.m = reinterpret_cast<float*>(p);
    v.s = reinterpret_cast<float*>(p + one);
    v.a = reinterpret_cast<int*>(p + 2 * one);
    return v;
}

inline size_t ws_size(int G, int B) { return 3 * align256(size_t(G) * B * 4); }

// Fold four logits (rows row0..row0+3, already in log2 units) into a state.
// Rows are visited in increasing order, so a strict '>' keeps the lowest
// index among equal maxima.
__device__ __forceinline__ void fold4(ArgSoft& st, const float x[4], int row0, int V) {
    float mx = st.m;
    int ax = st.a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (row0 + i < V && x[i] > mx) {
            mx = x[i];
            ax = row0 + i;
        }
    }
    float s = (st.s > 0.f) ? st.s * exp2f(st.m - mx) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (row0 + i < V) s += exp2f(x[i] - mx);
    st.m = mx;
    st.s = s;
    st.a = ax;
}

__device__ __forceinline__ ArgSoft shfl_xor_state(ArgSoft x, int off) {
    ArgSoft y;
    y.m = __shfl_xor(x.m, off);
    y.s = __shfl_xor(x.s, off);
    y.a = __shfl_xor(x.a, off);
    return y;
}

__device__ __forceinline__ void store_partial(const WsView& w, int G, int col, int part, ArgSoft s) {
    const size_t idx = size_t(col) * G + part;
    w.m[idx] = s.m;
    w.s[idx] = s.s;
    w.a[idx] = s.a;
}


// End of a streaming kernel: merge the four lane groups that hold the same
// position (lanes l, l^16, l^32, l^48), then the waves of the workgroup
// through `fin`, and store one partial state per position.
template <int NB>
__device__ __forceinline__ void store_workgroup_partials(ArgSoft (&st)[NB],
                                                         ArgSoft (*fin)[NB][16], void* ws,
                                                         int B) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        st[nb] = merge(st[nb], shfl_xor_state(st[nb], 16));
        st[nb] = merge(st[nb], shfl_xor_state(st[nb], 32));
        if (lane < 16) fin[wave][nb][lane] = st[nb];
    }
    __syncthreads();
    const int G = gridDim.x;
    const WsView wv = ws_view(ws, G, B);
    if (wave == 0 && lane < 16) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            ArgSoft s = fin[0][nb][lane];
            for (int w = 1; w < nwave; ++w) s = merge(s, fin[w][nb][lane]);
            const int col = nb * 16 + lane;
            if (col < B) store_partial(wv, G, col, blockIdx.x, s);
        }
    }
}

// Persistent grid for `ntiles` equal tiles.  The streaming kernels are bound
// by the aggregate HBM bandwidth, so their time follows the largest
// per-workgroup share, ceil(ntiles / G), times G.  Between 7/8 of the chip
// and all of it, take the grid that wastes the fewest tile slots (the largest
// such grid on ties): 9496 tiles, for instance, go 38 per workgroup to 250
// workgroups instead of 37 or 38 to 256, whose last twenty-four workgroups
// would run alone at the end.
inline int persistent_grid(int ntiles) {
    if (ntiles <= kMaxGrid) return ntiles;
    int best = kMaxGrid;
    long best_slots = long((ntiles + kMaxGrid - 1) / kMaxGrid) * kMaxGrid;
    for (int g = kMaxGrid - 1; g >= kMaxGrid - kMaxGrid / 8; --g) {
        const long slots = long((ntiles + g - 1) / g) * g;
        if (slots < best_slots) {
            best_slots = slots;
            best = g;
        }
    }
    return best;
}

// Merge of the partials written by a streaming kernel (and, with f.commit,
// the threshold commit), defined with the bf16 kernels.
hipError_t launch_combine(void* ws, int G, int B, const Finish& f, hipStream_t st);

}  // namespace bd
