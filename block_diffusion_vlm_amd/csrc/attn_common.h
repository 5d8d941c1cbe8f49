// Building blocks shared by the bf16 attention kernels (block attention over
// the KV cache and dual-stream training attention), on gfx950
// v_mfma_f32_32x32x16_bf16.
//
// Formulation.  A wave owns 32 query rows.  Scores are computed transposed,
// S^T[key][q] = K[key][:] . Q[q][:], with K as the A operand (read from LDS)
// and Q as the B operand (held in registers), and the output transposed as
// well, O^T[dh][q] = V^T[dh][key] . P^T[key][q], with V^T read from LDS and P
// taken straight from the score accumulators.  In the 32x32 accumulator layout
// lane l holds query column l % 32 for both products, so every per-row
// softmax quantity (max, sum, rescale factor) lives in the lane that needs it;
// only lanes l and l ^ 32 share a row.
//
// Accumulator layout (32x32, 16 floats per lane): register r of lane l holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.  Operand layout (A and B,
// 8 bf16 per lane): lane l holds row/column l % 32 and K indices
// 8*(l/32) .. 8*(l/32)+7.  For P^T the 16 keys of K-step s2 inside a 32-key
// block are taken from accumulator registers 8*s2 .. 8*s2+7, i.e. keys
// 16*s2 + 4*(l/32) + {0,1,2,3} and 16*s2 + 8 + 4*(l/32) + {0,1,2,3}; V^T is
// read with exactly that key permutation, so the sum over keys is unchanged.
#pragma once

#include "bd_internal.h"

namespace bd {
namespace attn {

constexpr int kDh = 128;           // head dimension of the bf16 kernels
constexpr int kBN = 64;            // keys per tile
constexpr int kKPitch = kDh + 8;   // LDS row pitch of K tiles (elements): 272 B
constexpr int kVPitch = kBN + 4;   // LDS row pitch of V^T tiles (elements): 136 B

struct Tiles {
    uint16_t k[kBN * kKPitch];      // K tile, [key][dh]
    uint16_t vt[kDh * kVPitch];     // V tile transposed, [dh][key]
};

// Key held by accumulator register r of lane l inside a 32-key block.
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// A 64-key tile of K and V in flight through registers: thread t holds keys
// t/16 + 16u (u = 0..3), dims 8*(t%16) .. +7, of both K and V.  256 threads.
struct TileRegs {
    u32x4 k[4];
    u32x4 v[4];
};

// Global -> registers for keys [j0, j0 + 64); keys at or beyond `jend` read
// as zeros.  `row_stride` is the distance between consecutive keys in elements.
__device__ __forceinline__ void fetch_tile(TileRegs& r, const uint16_t* __restrict__ kbase,
                                           const uint16_t* __restrict__ vbase, size_t row_stride,
                                           int j0, int jend) {
    const int tid = threadIdx.x;
    const int col = (tid & 15) * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = j0 + (tid >> 4) + 16 * u;
        r.k[u] = u32x4{0, 0, 0, 0};
        r.v[u] = u32x4{0, 0, 0, 0};
        if (j < jend) {
            r.k[u] = *reinterpret_cast<const u32x4*>(kbase + size_t(j) * row_stride + col);
            r.v[u] = *reinterpret_cast<const u32x4*>(vbase + size_t(j) * row_stride + col);
        }
    }
}

// Registers -> LDS: K as is, V transposed.
__device__ __forceinline__ void store_tile(Tiles& t, const TileRegs& r) {
    const int tid = threadIdx.x;
    const int col = (tid & 15) * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int key = (tid >> 4) + 16 * u;
        *reinterpret_cast<u32x4*>(&t.k[key * kKPitch + col]) = r.k[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t.vt[(col + 2 * e) * kVPitch + key] = static_cast<uint16_t>(r.v[u][e] & 0xFFFFu);
            t.vt[(col + 2 * e + 1) * kVPitch + key] = static_cast<uint16_t>(r.v[u][e] >> 16);
        }
    }
}

// Cooperative load of keys [j0, j0 + 64) of one head into LDS (K as is, V
// transposed).
__device__ __forceinline__ void load_tile(Tiles& t, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, size_t row_stride,
                                          int j0, int jend) {
    TileRegs r;
    fetch_tile(r, kbase, vbase, row_stride, j0, jend);
    store_tile(t, r);
}

// Q fragments (B operand of S^T) for 32 rows; rowptr == nullptr gives zeros.
__device__ __forceinline__ void load_q(bf16x8 (&qf)[8], const uint16_t* rowptr, int lane) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        u32x4 v = {0, 0, 0, 0};
        if (rowptr) v = *reinterpret_cast<const u32x4*>(rowptr + 16 * s + 8 * (lane >> 5));
        qf[s] = __builtin_bit_cast(bf16x8, v);
    }
}

// S^T for the 64 keys of a tile: sacc[kb] covers keys 32*kb .. 32*kb+31.
__device__ __forceinline__ void scores(f32x16 (&sacc)[2], const Tiles& t, const bf16x8 (&qf)[8],
                                       int lane) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x16 acc = {};
        const uint16_t* kr = &t.k[(32 * kb + (lane & 31)) * kKPitch + 8 * (lane >> 5)];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * s));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc, 0, 0, 0);
        }
        sacc[kb] = acc;
    }
}

// O^T += V^T P^T for one tile; p[kb][r] are the probabilities of the keys in
// sacc layout.
__device__ __forceinline__ void accumulate_pv(f32x16 (&oacc)[4], const Tiles& t,
                                              const float (&p)[2][16], int lane) {
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[kb][8 * s2 + 2 * e], p[kb][8 * s2 + 2 * e + 1]);
            pf[kb][s2] = __builtin_bit_cast(bf16x8, w);
        }
    const int g4 = 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const uint16_t* vr = &t.vt[(32 * db + (lane & 31)) * kVPitch];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int key0 = 32 * kb + 16 * s2 + g4;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + key0);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + key0 + 8);
                const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), pf[kb][s2], oacc[db], 0, 0, 0);
            }
    }
}

}  // namespace attn
}  // namespace bd
