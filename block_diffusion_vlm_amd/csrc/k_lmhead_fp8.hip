// FP8 (W8A8) LM-head confidence.  W is stored as OCP E4M3 codes [V][d] with
// one float32 scale per vocabulary row (per-output-channel weights, as in
// SmoothQuant W8A8: Fast-dVLM overview §2.3.2); the hidden states (bf16) are
// quantized per position when the kernel starts (per-token dynamic
// activations):
//   amax = max_k |h[k]|,  r = 448 / amax,  s_h = amax / 448   (float32;
//   r = s_h = 1 for an all-zero row),
//   code_k = E4M3(clamp(h[k] * r, -448, 448)), rounded to nearest even,
//   l[v] = s_h * s_w[v] * sum_k code_k(h) code_k(W[v])   (float32 sums).
// Then the same split-vocabulary softmax maximum as the bf16 path: partial
// (max, sum, argmax) states per workgroup, merged by launch_combine.
//
// The contraction runs on v_mfma_f32_16x16x128_f8f6f4 with both operands in
// E4M3: the codes go from LDS straight into the A operand, with no
// conversion.  The K order inside a 128-byte chunk is the same for A and B
// (lane group g, byte t <-> k = 32g + t), which leaves the dot product
// unchanged.  Compared with bf16 the weights take half the bytes, so the
// kernel streams twice the vocabulary per byte of HBM traffic.
#include "lmhead_common.h"

namespace bd {

namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4m3Max = 448.0f;
constexpr int kFp8Rows = 32;   // vocabulary rows per tile (two 16-row MFMA blocks)

struct RowQuant {
    float r;   // multiplier into the code domain
    float s;   // dequantization scale
};

__device__ __forceinline__ RowQuant row_quant(float amax) {
    if (amax > 0.f) return RowQuant{kE4m3Max / amax, amax / kE4m3Max};
    return RowQuant{1.f, 1.f};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Largest magnitude among eight bf16 values.
__device__ __forceinline__ float absmax8(u32x4 v) {
    float m = fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x)));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
    return m;
}

// Four bf16 values (two dwords, element order low half first) -> four E4M3
// codes in one dword (byte i = element i).  The product is clamped to the
// format's range first (it can exceed 448 by an ulp); the conversion rounds
// to nearest even.
__device__ __forceinline__ uint32_t quant4(uint32_t w01, uint32_t w23, float r) {
    const float a0 = __builtin_amdgcn_fmed3f(bf16_lo(w01) * r, kE4m3Max, -kE4m3Max);
    const float a1 = __builtin_amdgcn_fmed3f(bf16_hi(w01) * r, kE4m3Max, -kE4m3Max);
    const float a2 = __builtin_amdgcn_fmed3f(bf16_lo(w23) * r, kE4m3Max, -kE4m3Max);
    const float a3 = __builtin_amdgcn_fmed3f(bf16_hi(w23) * r, kE4m3Max, -kE4m3Max);
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, c, true);
    return static_cast<uint32_t>(c);
}

__device__ __forceinline__ u32x2 quant8(u32x4 v, float r) {
    return u32x2{quant4(v.x, v.y, r), quant4(v.z, v.w, r)};
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
    // Format selectors 0/0: both operands E4M3.  Zero scale operands select
    // the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Scales of vocabulary rows r0 .. r0+3 (r0 a multiple of 4), clamped to the
// last row at the tail.
__device__ __forceinline__ f32x4 load_scales4(const float* __restrict__ ws, int r0, int V) {
    if (r0 + 3 < V) return *reinterpret_cast<const f32x4*>(ws + r0);
    f32x4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = ws[r0 + i < V ? r0 + i : V - 1];
    return s;
}

// ---------------------------------------------------------------------------
// Row quantizer: one workgroup per row, the rule above.  Used for stored
// weights (bd_quant_fp8_rows) and for the hidden states of the generic
// LM-head path.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int d,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale,
                                                         const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    __shared__ float wmax[4];
    const size_t row = blockIdx.x;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * d);
    const int n8 = d / 8;
    float m = 0.f;
    for (int i = threadIdx.x; i < n8; i += 256) m = fmaxf(m, absmax8(xr[i]));
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const RowQuant rq = row_quant(amax);
    u32x2* qr = reinterpret_cast<u32x2*>(q + row * d);
    for (int i = threadIdx.x; i < n8; i += 256) qr[i] = quant8(xr[i], rq.r);
    if (threadIdx.x == 0) scale[row] = rq.s;
}

// ---------------------------------------------------------------------------
// Streaming kernel.  NB = ceil(B/16) position blocks, NCH = 128-byte K chunks
// per wave; blockDim.x = 64 * ks and d = 128 * NCH * ks.
//
// Wave w owns K range [w*NCH*128, (w+1)*NCH*128) of every 32-row tile: a
// 32-row x NCH*128-byte region, read with 4*NCH non-temporal 16-byte loads
// per lane (consecutive lanes read consecutive 16-byte pieces of a row),
// staged in a wave-private LDS buffer, and read back as A operands.  Row r's
// piece p sits in slot p ^ (r & SW), so the 16 rows of one operand read fall
// in distinct banks.  Two tiles are in flight in registers (with their 32
// row scales each) while the current tile is multiplied: the tiles carry
// half the bytes of the bf16 kernel's, so one tile ahead does not cover the
// memory latency.  The waves add their partial logits through LDS; one wave
// (rotating) scales them and folds them into the running states.
//
// Prologue: each wave loads its K range of h, the workgroup takes the row
// maxima (lane groups by shuffles, waves through LDS), and each lane keeps
// the E4M3 B operands of its rows for the whole kernel.
// ---------------------------------------------------------------------------
template <int NB, int NCH, int DEPTH = 2>
__global__ __launch_bounds__(256) void lmhead_fp8_kernel(const uint16_t* __restrict__ h,
                                                         const uint8_t* __restrict__ W,
                                                         const float* __restrict__ wscale, int B,
                                                         int d, int V, int ntiles,
                                                         void* __restrict__ ws,
                                                         const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    constexpr int RT = kFp8Rows / 16;              // MFMA row blocks per tile
    constexpr int PIECES = NCH * 8;                // 16-byte pieces per row segment
    constexpr int NL = kFp8Rows * PIECES / 64;     // 16-byte loads per lane per tile
    constexpr int SW = (PIECES % 16 == 0) ? 15 : 7;
    __shared__ f32x4 red[2][4][RT][NB][64];        // per-wave partial logits, 2 buffers
    __shared__ ArgSoft fin[4][NB][16];
    __shared__ float amx[4][NB * 16];
    __shared__ __align__(16) u32x4 stage[4][kFp8Rows * PIECES];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int kw = wave * NCH * 128;               // this wave's K start (elements = bytes)
    const int G = gridDim.x;

    // Load i of a lane covers slot q = 64 i + lane of the row-major
    // [32 rows][PIECES] region: row q / PIECES, slot q % PIECES, holding
    // piece (slot ^ (row & SW)).
    auto load_tile = [&](u32x4 (&buf)[NL], int tile) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int q = 64 * i + lane;
            const int r = q / PIECES;
            const int piece = (q % PIECES) ^ (r & SW);
            int row = tile * kFp8Rows + r;
            row = row < V ? row : V - 1;
            buf[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(W + size_t(row) * d + kw) + piece);
        }
    };
    auto load_scales = [&](f32x4 (&sc)[RT], int tile) {
#pragma unroll
        for (int s = 0; s < RT; ++s) sc[s] = load_scales4(wscale, tile * kFp8Rows + s * 16 + g * 4, V);
    };

    const int t_beg = int(int64_t(ntiles) * blockIdx.x / G);
    const int t_end = int(int64_t(ntiles) * (blockIdx.x + 1) / G);
    u32x4 bufA[NL], bufB[NL];                      // DEPTH (1 or 2) tiles in flight
    f32x4 scA[RT], scB[RT];
    auto issue_first_tiles = [&]() {
        if (t_beg < t_end) {
            load_tile(bufA, t_beg);
            load_scales(scA, t_beg);
        }
        if constexpr (DEPTH == 2) {
            if (t_beg + 1 < t_end) {
                load_tile(bufB, t_beg + 1);
                load_scales(scB, t_beg + 1);
            }
        }
    };

    // ---- quantize h: lane (r16, g) holds k = kw + 128c + 32g + [0, 32) of
    // position nb*16 + r16, as 32 codes (8 dwords, byte t <-> k offset t).
    // The h loads are issued before the first tiles' loads (loads return in
    // order), so the quantization runs while those tiles are in flight; when
    // the raw values would take too many registers, h is read twice, both
    // times before the tiles.
    auto h_piece = [&](int nb, int c, int j) -> u32x4 {
        const int row = nb * 16 + r16;
        if (row >= B) return u32x4{0, 0, 0, 0};
        return reinterpret_cast<const u32x4*>(h + size_t(row) * d + kw + c * 128 + g * 32)[j];
    };
    auto row_amax = [&](float (&m)[NB]) -> void {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m[nb] = fmaxf(m[nb], __shfl_xor(m[nb], 16));
            m[nb] = fmaxf(m[nb], __shfl_xor(m[nb], 32));
            if (g == 0) amx[wave][nb * 16 + r16] = m[nb];
        }
        __syncthreads();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float amax = amx[0][nb * 16 + r16];
            for (int w = 1; w < nwave; ++w) amax = fmaxf(amax, amx[w][nb * 16 + r16]);
            m[nb] = amax;
        }
    };
    float shl[NB];                                 // s_h * log2(e) of this lane's position
    i32x8 hq[NCH][NB];
    auto put_codes = [&](int c, int nb, int j, u32x2 q) {
        hq[c][nb][2 * j] = static_cast<int32_t>(q.x);
        hq[c][nb][2 * j + 1] = static_cast<int32_t>(q.y);
    };
    float m[NB];
    if constexpr (NCH * NB <= 4) {
        u32x4 raw[NCH][NB][4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) raw[c][nb][j] = h_piece(nb, c, j);
        issue_first_tiles();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m[nb] = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) m[nb] = fmaxf(m[nb], absmax8(raw[c][nb][j]));
        }
        row_amax(m);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const RowQuant rq = row_quant(m[nb]);
            shl[nb] = rq.s * kLog2e;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) put_codes(c, nb, j, quant8(raw[c][nb][j], rq.r));
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m[nb] = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) m[nb] = fmaxf(m[nb], absmax8(h_piece(nb, c, j)));
        }
        row_amax(m);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const RowQuant rq = row_quant(m[nb]);
            shl[nb] = rq.s * kLog2e;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) put_codes(c, nb, j, quant8(h_piece(nb, c, j), rq.r));
        }
        issue_first_tiles();
    }

    ArgSoft st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st[nb] = ArgSoft{-INFINITY, 0.f, 0x7fffffff};

    // One tile: stage it, refill its register buffer with the tile two
    // ahead, multiply, reduce across the waves, fold.
    int it = 0;
    auto step = [&](u32x4 (&buf)[NL], f32x4 (&scb)[RT], int tile) {
        // The previous tile's operand reads precede these writes in this
        // wave's program order, so the wave-private buffer can be refilled.
#pragma unroll
        for (int i = 0; i < NL; ++i) stage[wave][64 * i + lane] = buf[i];
        f32x4 sc[RT];
#pragma unroll
        for (int s = 0; s < RT; ++s) sc[s] = scb[s];
        if (tile + DEPTH < t_end) {
            load_tile(buf, tile + DEPTH);
            load_scales(scb, tile + DEPTH);
        }

        f32x4 acc[RT][NB];
#pragma unroll
        for (int s = 0; s < RT; ++s)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < RT; ++s) {
            const int r = s * 16 + r16;
            const u32x4* srow = &stage[wave][r * PIECES];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int p0 = c * 8 + 2 * g;
                const u32x4 lo = srow[p0 ^ (r & SW)];
                const u32x4 hi = srow[(p0 + 1) ^ (r & SW)];
                const i32x8 a = {int32_t(lo.x), int32_t(lo.y), int32_t(lo.z), int32_t(lo.w),
                                 int32_t(hi.x), int32_t(hi.y), int32_t(hi.z), int32_t(hi.w)};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[s][nb] = mfma_fp8(a, hq[c][nb], acc[s][nb]);
            }
        }

        bool mine = true;
        if (nwave > 1) {
#pragma unroll
            for (int s = 0; s < RT; ++s)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) red[it & 1][wave][s][nb][lane] = acc[s][nb];
            __syncthreads();
            mine = (wave == it % nwave);
            if (mine) {
#pragma unroll
                for (int s = 0; s < RT; ++s)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        f32x4 t = red[it & 1][0][s][nb][lane];
                        for (int w = 1; w < nwave; ++w) t += red[it & 1][w][s][nb][lane];
                        acc[s][nb] = t;
                    }
            }
        }
        if (mine) {
#pragma unroll
            for (int s = 0; s < RT; ++s) {
                const int row0 = tile * kFp8Rows + s * 16 + g * 4;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float x[4] = {acc[s][nb][0] * sc[s][0] * shl[nb],
                                        acc[s][nb][1] * sc[s][1] * shl[nb],
                                        acc[s][nb][2] * sc[s][2] * shl[nb],
                                        acc[s][nb][3] * sc[s][3] * shl[nb]};
                    fold4(st[nb], x, row0, V);
                }
            }
        }
        ++it;
    };
    if constexpr (DEPTH == 2) {
        for (int tile = t_beg; tile < t_end; tile += 2) {
            step(bufA, scA, tile);
            if (tile + 1 < t_end) step(bufB, scB, tile + 1);
        }
    } else {
        for (int tile = t_beg; tile < t_end; ++tile) step(bufA, scA, tile);
    }

    store_workgroup_partials<NB>(st, fin, ws, B);
}

// Generic FP8 kernel for shapes whose operands do not fit the streaming
// kernel's registers and LDS (large B x d): the hidden states are quantized
// into the workspace first (quant_rows_kernel); one wave per 32-row tile runs
// over the whole K range and re-reads the (cached) hidden codes per chunk.
template <int NB>
__global__ __launch_bounds__(256) void lmhead_fp8_generic_kernel(
    const uint8_t* __restrict__ hq, const float* __restrict__ hs, const uint8_t* __restrict__ W,
    const float* __restrict__ wscale, int B, int d, int V, int ntiles, void* __restrict__ ws,
    const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    __shared__ ArgSoft fin[4][NB][16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int G = gridDim.x;

    float shl[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + r16;
        shl[nb] = (col < B ? hs[col] : 1.f) * kLog2e;
    }
    ArgSoft st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st[nb] = ArgSoft{-INFINITY, 0.f, 0x7fffffff};

    for (int tile = blockIdx.x * nwave + wave; tile < ntiles; tile += G * nwave) {
#pragma unroll
        for (int s = 0; s < kFp8Rows / 16; ++s) {
            int row = tile * kFp8Rows + s * 16 + r16;
            row = row < V ? row : V - 1;
            const u32x4* wp = reinterpret_cast<const u32x4*>(W + size_t(row) * d + g * 32);
            f32x4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < d / 128; ++c) {
                const u32x4 lo = wp[c * 8];
                const u32x4 hi = wp[c * 8 + 1];
                const i32x8 a = {int32_t(lo.x), int32_t(lo.y), int32_t(lo.z), int32_t(lo.w),
                                 int32_t(hi.x), int32_t(hi.y), int32_t(hi.z), int32_t(hi.w)};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int col = nb * 16 + r16;
                    u32x4 blo = u32x4{0, 0, 0, 0}, bhi = u32x4{0, 0, 0, 0};
                    if (col < B) {
                        const u32x4* hp =
                            reinterpret_cast<const u32x4*>(hq + size_t(col) * d + g * 32);
                        blo = hp[c * 8];
                        bhi = hp[c * 8 + 1];
                    }
                    const i32x8 b = {int32_t(blo.x), int32_t(blo.y), int32_t(blo.z),
                                     int32_t(blo.w), int32_t(bhi.x), int32_t(bhi.y),
                                     int32_t(bhi.z), int32_t(bhi.w)};
                    acc[nb] = mfma_fp8(a, b, acc[nb]);
                }
            }
            const int row0 = tile * kFp8Rows + s * 16 + g * 4;
            const f32x4 sc = load_scales4(wscale, row0, V);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float x[4] = {acc[nb][0] * sc[0] * shl[nb], acc[nb][1] * sc[1] * shl[nb],
                                    acc[nb][2] * sc[2] * shl[nb], acc[nb][3] * sc[3] * shl[nb]};
                fold4(st[nb], x, row0, V);
            }
        }
    }
    store_workgroup_partials<NB>(st, fin, ws, B);
}

// Host plan of the streaming kernel: waves per workgroup (K split) and
// chunks per wave, within the register and LDS budget (NCH * (2 + NB) <= 24
// and NB + NCH <= 9 keep the staging buffers, the reduction buffers and the
// operands within one workgroup per CU).  Returns false when only the generic
// kernel applies.
bool plan_fp8(int B, int d, int* ks, int* nch) {
    const int NB = (B + 15) / 16;
    const int c = d / 128;
    const int order[3] = {4, 2, 1};
    for (int i = 0; i < 3; ++i) {
        const int k = order[i];
        if (c % k != 0) continue;
        const int n = c / k;
        if (n <= 8 && n * (2 + NB) <= 24 && NB + n <= 9) {
            *ks = k;
            *nch = n;
            return true;
        }
    }
    return false;
}

// Workspace: the partial states, then (generic path) the hidden codes and
// their scales.
struct Fp8Ws {
    size_t partial_bytes;
    size_t codes_off;
    size_t scales_off;
    size_t total;
};

Fp8Ws fp8_ws_layout(int B, int d, int V) {
    Fp8Ws L;
    L.partial_bytes = ws_size(lmhead_fp8_grid(B, d, V), B);
    L.codes_off = align256(L.partial_bytes);
    L.scales_off = L.codes_off + align256(size_t(B) * d);
    L.total = L.scales_off + align256(size_t(B) * 4);
    return L;
}

template <int NB, int NCH>
void launch_fp8_stream(int G, int ks, const uint16_t* h, const uint8_t* W, const float* wsc,
                       int B, int d, int V, int ntiles, void* ws, hipStream_t st,
                       const int32_t* gate) {
    // Two tiles in flight for one position block; one for more, whose
    // hidden codes and accumulators would otherwise push the second tile's
    // registers out to the accumulation registers.
    constexpr int kDepth = NB == 1 ? 2 : 1;
    hipLaunchKernelGGL((lmhead_fp8_kernel<NB, NCH, kDepth>), dim3(G), dim3(64 * ks), 0, st, h, W,
                       wsc, B, d, V, ntiles, ws, gate);
}

template <int NB>
hipError_t launch_fp8_nb(const void* h, const uint8_t* W, const float* wsc, int B, int d, int V,
                         const Finish& f, void* ws, hipStream_t st) {
    const int ntiles = (V + kFp8Rows - 1) / kFp8Rows;
    const int G = lmhead_fp8_grid(B, d, V);
    const auto* hh = static_cast<const uint16_t*>(h);
    int ks = 0, nch = 0;
    if (!plan_fp8(B, d, &ks, &nch)) {
        const Fp8Ws L = fp8_ws_layout(B, d, V);
        uint8_t* base = static_cast<uint8_t*>(ws);
        uint8_t* hq = base + L.codes_off;
        float* hs = reinterpret_cast<float*>(base + L.scales_off);
        hipLaunchKernelGGL(quant_rows_kernel, dim3(B), dim3(256), 0, st, hh, d, hq, hs, f.gate);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(lmhead_fp8_generic_kernel<NB>, dim3(G), dim3(256), 0, st, hq, hs, W,
                           wsc, B, d, V, ntiles, ws, f.gate);
        e = hipGetLastError();
        return e != hipSuccess ? e : launch_combine(ws, G, B, f, st);
    }
    // Combinations that plan_fp8 never selects are not instantiated.
#define BD_FP8_CASE(N)                                                               \
    case N:                                                                          \
        if constexpr (N * (2 + NB) <= 24 && NB + N <= 9) {                           \
            launch_fp8_stream<NB, N>(G, ks, hh, W, wsc, B, d, V, ntiles, ws, st, f.gate); \
        } else {                                                                     \
            return hipErrorInvalidValue;                                             \
        }                                                                            \
        break;
    switch (nch) {
        BD_FP8_CASE(1)
        BD_FP8_CASE(2)
        BD_FP8_CASE(3)
        BD_FP8_CASE(4)
        BD_FP8_CASE(5)
        BD_FP8_CASE(6)
        BD_FP8_CASE(7)
        BD_FP8_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef BD_FP8_CASE
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine(ws, G, B, f, st);
}

}  // namespace

int lmhead_fp8_grid(int B, int d, int V) {
    (void)B;
    (void)d;
    return persistent_grid((V + kFp8Rows - 1) / kFp8Rows);
}

size_t lmhead_fp8_ws_bytes(int B, int d, int V) { return fp8_ws_layout(B, d, V).total; }

hipError_t launch_lmhead_fp8(const void* h, const uint8_t* W, const float* w_scale, int B, int d,
                             int V, const Finish& f, void* ws, hipStream_t st) {
    switch ((B + 15) / 16) {
        case 1: return launch_fp8_nb<1>(h, W, w_scale, B, d, V, f, ws, st);
        case 2: return launch_fp8_nb<2>(h, W, w_scale, B, d, V, f, ws, st);
        case 3: return launch_fp8_nb<3>(h, W, w_scale, B, d, V, f, ws, st);
        case 4: return launch_fp8_nb<4>(h, W, w_scale, B, d, V, f, ws, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quant_fp8_rows(const void* x, int R, int d, uint8_t* q, float* scale,
                                 hipStream_t st) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_rows_kernel, dim3(R), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), d, q, scale, nullptr);
    return hipGetLastError();
}

}  // namespace bd
