// Building blocks shared by the bf16 attention kernels (block attention over
// the KV cache and dual-stream training attention), on gfx950
// v_mfma_f32_32x32x16_bf16.
//
// Formulation.  A wave owns RB blocks of 32 query rows.  Scores are computed
// transposed, S^T[key][q] = K[key][:] . Q[q][:], with K as the A operand (read
// from LDS) and Q as the B operand (held in registers), and the output
// transposed as well, O^T[dh][q] = V^T[dh][key] . P^T[key][q], with V^T read
// from LDS by transposing loads and P taken straight from the score
// accumulators.  In the 32x32 accumulator layout lane l holds query column
// l % 32 for both products, so every per-row softmax quantity (max, sum,
// rescale factor) lives in the lane that needs it; only lanes l and l ^ 32
// share a row.  Each A fragment read from LDS feeds RB MFMAs.
//
// Accumulator layout (32x32, 16 floats per lane): register r of lane l holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.  Operand layout (A and B,
// 8 bf16 per lane): lane l holds row/column l % 32 and K indices
// 8*(l/32) .. 8*(l/32)+7.  For P^T the 16 keys of K-step s2 inside a 32-key
// block are taken from accumulator registers 8*s2 .. 8*s2+7, i.e. keys
// 16*s2 + 4*(l/32) + {0,1,2,3} and 16*s2 + 8 + 4*(l/32) + {0,1,2,3}; V^T is
// read with exactly that key permutation, so the sum over keys is unchanged.
//
// LDS tiles.  K and V are both stored row-major ([key][dh]) with 16-byte
// stores.  K rows are padded to 272 bytes, so the 16 keys of one fragment
// load fall in distinct banks.  V^T fragments come from ds_read_b64_tr_b16:
// within each 16-lane group, lane i of the result receives element
// (i % 4) of the 8 bytes addressed by lane 4k + i/4, for k = 0..3; with lane
// L addressing V[key0 + L/4][dh0 + 4 (L%4)], lane i therefore receives
// V[key0 + k][dh0 + i], k = 0..3 - four keys of one dh column.  V rows are
// padded to 288 bytes, so the four rows read by one group use distinct banks.
#pragma once

#include "bd_internal.h"

#define BD_LDS __attribute__((address_space(3)))

namespace bd {
namespace attn {

constexpr int kDh = 128;           // head dimension of the bf16 kernels
constexpr int kBN = 64;            // keys per tile
constexpr int kKPitch = kDh + 8;   // LDS row pitch of K tiles (elements): 272 B
constexpr int kVPitch = kDh + 16;  // LDS row pitch of V tiles (elements): 288 B

struct Tiles {
    uint16_t k[kBN * kKPitch];      // K tile, [key][dh]
    uint16_t v[kBN * kVPitch];      // V tile, [key][dh]
};

// Key held by accumulator register r of lane l inside a 32-key block.
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// A 64-key tile of K and V in flight through registers.  With T threads,
// thread t holds 16-byte pieces p = t + T u (u < 1024 / T) of both K and V:
// key p / 16, dims 8 (p % 16) .. +7.
template <int T>
struct TileRegs {
    static constexpr int N = 1024 / T;
    u32x4 k[N];
    u32x4 v[N];
};

// Global -> registers for keys [j0, j0 + 64); keys at or beyond `jend` read
// as zeros.  `row_stride` is the distance between consecutive keys in elements.
template <int T>
__device__ __forceinline__ void fetch_tile(TileRegs<T>& r, const uint16_t* __restrict__ kbase,
                                           const uint16_t* __restrict__ vbase, size_t row_stride,
                                           int j0, int jend) {
    constexpr int KEYS_PER_U = T / 16;               // key rows between consecutive u
    const int key = threadIdx.x >> 4;
    const int col = (threadIdx.x & 15) * 8;
    const size_t off = size_t(j0 + key) * row_stride + col;
    const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off);
    const size_t step = size_t(KEYS_PER_U) * row_stride / 8;   // in 16-byte units
    if (j0 + kBN <= jend) {
#pragma unroll
        for (int u = 0; u < TileRegs<T>::N; ++u) {
            r.k[u] = kp[u * step];
            r.v[u] = vp[u * step];
        }
    } else {
#pragma unroll
        for (int u = 0; u < TileRegs<T>::N; ++u) {
            const bool ok = j0 + key + KEYS_PER_U * u < jend;
            r.k[u] = ok ? kp[u * step] : u32x4{0, 0, 0, 0};
            r.v[u] = ok ? vp[u * step] : u32x4{0, 0, 0, 0};
        }
    }
}

// Registers -> LDS (both row-major).
template <int T>
__device__ __forceinline__ void store_tile(Tiles& t, const TileRegs<T>& r) {
#pragma unroll
    for (int u = 0; u < TileRegs<T>::N; ++u) {
        const int p = threadIdx.x + T * u;
        const int key = p >> 4;
        const int col = (p & 15) * 8;
        *reinterpret_cast<u32x4*>(&t.k[key * kKPitch + col]) = r.k[u];
        *reinterpret_cast<u32x4*>(&t.v[key * kVPitch + col]) = r.v[u];
    }
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

// S^T for the 64 keys of a tile and RB row blocks: sacc[rb][kb] covers keys
// 32*kb .. 32*kb+31 of row block rb.
template <int RB>
__device__ __forceinline__ void scores(f32x16 (&sacc)[RB][2], const Tiles& t,
                                       const bf16x8 (&qf)[RB][8], int lane) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = f32x16{};
        const uint16_t* kr = &t.k[(32 * kb + (lane & 31)) * kKPitch + 8 * (lane >> 5)];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * s));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                sacc[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][s], sacc[rb][kb],
                                                                       0, 0, 0);
        }
    }
}

// Transposing LDS load of four keys of one dh column (see the file comment).
__device__ __forceinline__ bf16x4 read_vt4(const uint16_t* p) {
    typedef __bf16 lds_bf16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (BD_LDS lds_bf16x4*)(const_cast<uint16_t*>(p)));
}

// bf16 P^T fragments of one tile from probabilities in score-accumulator
// order: pf[rb][kb][s2] = p[rb][kb][8*s2 .. 8*s2+7].  The probabilities live
// in their own registers, never in the MFMA accumulators: VALU writes into
// registers that an MFMA chain also writes are avoided altogether.
template <int RB>
__device__ __forceinline__ void pack_p(bf16x8 (&pf)[RB][2][2], const float (&sacc)[RB][2][16]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pf[rb][kb][s2][e] = static_cast<__bf16>(sacc[rb][kb][8 * s2 + e]);
}

// O^T += V^T P^T for one tile.
template <int RB>
__device__ __forceinline__ void accumulate_pv(f32x16 (&oacc)[RB][4], const Tiles& t,
                                              const bf16x8 (&pf)[RB][2][2], int lane) {
    // Supplier lane L of 16-lane group q addresses V[key0 + L/4][dh0 + 4 (L%4)]
    // with key0 = 32 kb + 16 s2 + 4 (q / 2) (+ 8 for the upper four keys) and
    // dh0 = 32 db + 16 (q % 2).
    const int q = lane >> 4;
    const int L = lane & 15;
    const uint16_t* vbase = &t.v[(4 * (q >> 1) + (L >> 2)) * kVPitch + 16 * (q & 1) + 4 * (L & 3)];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint16_t* vp = vbase + (32 * kb + 16 * s2) * kVPitch + 32 * db;
                const bf16x4 lo = read_vt4(vp);
                const bf16x4 hi = read_vt4(vp + 8 * kVPitch);
                const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb][kb][s2],
                                                                           oacc[rb][db], 0, 0, 0);
            }
}

}  // namespace attn
}  // namespace bd
