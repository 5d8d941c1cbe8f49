// LM-head confidence: logits = h W^T fused with a split-vocabulary softmax
// maximum, so no logit ever reaches memory.  Per position b it yields the
// argmax token and conf = max_w p(w) = 1 / sum_v exp(l_v - max l) (the anchor
// confidence of the LOWN article, 'method step details' (1)).
//
// bf16 path (gfx950 MFMA).  The contraction is W[V][d] x h^T[d][B] with the
// vocabulary as the M dimension and the positions as N, on
// v_mfma_f32_16x16x32_bf16.  W is streamed exactly once, straight from HBM
// with non-temporal loads and staged through LDS into the A operand (see the
// kernel).  The K index inside a 128-element chunk is permuted identically
// for A and B (lane group g, MFMA j, element e <-> k = 32g + 8j + e), which
// leaves the dot product unchanged.  h is tiny and is held in registers as
// ready-made B fragments for the wave's K range.
//
// A workgroup has `ks` waves that split K; per 16-row vocabulary tile they
// add their partial logits through LDS and one wave (rotating; a different
// wave for each 16-position block) folds the 16 rows into running (max, sum,
// argmax) states in the log2 domain.  Each
// workgroup of a persistent grid streams one contiguous range of tiles (the
// ranges differ by at most one tile).  Each workgroup writes one partial state per position;
// a second, small kernel (one wave per position) merges the partials in a
// fixed order, so the result is deterministic; the same merge, followed by
// the threshold commit, runs as a single workgroup when the caller asks for
// both.  The kernel boundary makes
// the partials visible to the merge; an in-kernel "last workgroup" merge
// would need a device-scope release fence per workgroup, which on gfx950
// writes back the L2 and costs far more than the second launch.
#include "commit_impl.h"
#include "lmhead_common.h"

namespace bd {

namespace {

// Merge of the G partial states of one position by one wave, in a fixed
// order: lane l folds partials l, l + 64, ... .  They are read 512 at a time
// (eight per lane, every load of a batch issued before the first fold, so a
// batch costs one memory round trip), then a fixed xor-shuffle tree merges
// the lanes.  The result is valid in every lane.
__device__ ArgSoft reduce_column(const WsView& w, int G, int col) {
    const int lane = threadIdx.x & 63;
    const float* m = w.m + size_t(col) * G;
    const float* s = w.s + size_t(col) * G;
    const int* a = w.a + size_t(col) * G;
    ArgSoft st{-INFINITY, 0.f, 0x7fffffff};
    for (int p0 = 0; p0 < G; p0 += 8 * 64) {
        float mm[8], ss[8];
        int aa[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // Past the last partial: reload the last one and drop it below.
            const int p = min(p0 + 64 * u + lane, G - 1);
            mm[u] = m[p];
            ss[u] = s[p];
            aa[u] = a[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (p0 + 64 * u + lane >= G) mm[u] = -INFINITY, ss[u] = 0.f, aa[u] = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < 8; ++u) st = merge(st, ArgSoft{mm[u], ss[u], aa[u]});
    }
    for (int off = 1; off < 64; off <<= 1) st = merge(st, shfl_xor_state(st, off));
    return st;
}

// reduce_column for a group of LANES lanes (64, 32 or 16) of a wave, so that
// the 64 / LANES groups of a wave merge as many positions side by side: lane
// l of the group folds partials l, l + LANES, ..., eight per batch with every
// load of a batch issued first, then a fixed xor-shuffle tree inside the
// group (offsets below LANES never leave it).  The result is valid in every
// lane of the group; with LANES = 64 it is reduce_column, bit for bit.
template <int LANES>
__device__ ArgSoft reduce_column_lanes(const WsView& w, int G, int col) {
    const int gl = threadIdx.x & (LANES - 1);
    const float* m = w.m + size_t(col) * G;
    const float* s = w.s + size_t(col) * G;
    const int* a = w.a + size_t(col) * G;
    ArgSoft st{-INFINITY, 0.f, 0x7fffffff};
    for (int p0 = 0; p0 < G; p0 += 8 * LANES) {
        float mm[8], ss[8];
        int aa[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // Past the last partial: reload the last one and drop it below.
            const int p = min(p0 + LANES * u + gl, G - 1);
            mm[u] = m[p];
            ss[u] = s[p];
            aa[u] = a[p];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (p0 + LANES * u + gl >= G) mm[u] = -INFINITY, ss[u] = 0.f, aa[u] = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < 8; ++u) st = merge(st, ArgSoft{mm[u], ss[u], aa[u]});
    }
    for (int off = 1; off < LANES; off <<= 1) st = merge(st, shfl_xor_state(st, off));
    return st;
}

// One workgroup of 16 waves merges every position, 16 x 64 / LANES at a time
// (LANES = 64 up to 16 positions, 32 up to 32, 16 up to 64: a single round
// for any B), then wave 0 runs the speculative accept of the first accept_B
// positions against the draft tokens (Fast-dVLM overview §2.3.1), so the
// accept needs no dispatch of its own.
template <int LANES>
__global__ __launch_bounds__(1024) void lmhead_combine_accept_kernel(
    const void* __restrict__ ws, int G, int B, float* __restrict__ conf,
    int32_t* __restrict__ argmax, const int32_t* __restrict__ draft, int B_acc, int P,
    int bonus, int32_t* __restrict__ accepted, int32_t* __restrict__ kv_len,
    int32_t* __restrict__ out_tokens) {
    constexpr int kPerWave = 64 / LANES;
    __shared__ int sarg[64];
    const WsView w = ws_view(const_cast<void*>(ws), G, B);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    // The draft tokens are read now, with the partials (every wave reads
    // them, unconditionally, so no branch waits on them).
    const int32_t d = draft[min(lane, B_acc - 1)];
    for (int c0 = wave * kPerWave; c0 < B; c0 += 16 * kPerWave) {
        const int col = c0 + lane / LANES;
        const ArgSoft r = reduce_column_lanes<LANES>(w, G, min(col, B - 1));
        if ((lane & (LANES - 1)) == 0 && col < B) {
            conf[col] = 1.0f / r.s;
            argmax[col] = r.a;
            sarg[col] = r.a;
        }
    }
    __syncthreads();
    if (wave == 0)
        accept_wave(bonus != 0, d, lane < B_acc ? sarg[lane] : 0, B_acc, P, accepted, kv_len,
                    out_tokens);
}

// One wave per position: merged confidence and argmax.  As the AR seed of a
// block (seed_B > 0, one position), it also starts the block: argmax points
// at the block's tokens, so position 0 receives the seed token; positions
// 1 .. seed_B - 1 get token 0 and are masked, and the gate of the block's
// steps is seed_B - 1.
__global__ __launch_bounds__(64) void lmhead_combine_kernel(const void* __restrict__ ws, int G,
                                                            int B, float* __restrict__ conf,
                                                            int32_t* __restrict__ argmax,
                                                            const int32_t* __restrict__ gate,
                                                            int seed_B,
                                                            uint8_t* __restrict__ seed_masked,
                                                            int32_t* __restrict__ gate_out) {
    if (gated_off(gate)) return;
    const WsView w = ws_view(const_cast<void*>(ws), G, B);
    const int col = blockIdx.x;
    const ArgSoft r = reduce_column(w, G, col);
    if (threadIdx.x == 0) {
        conf[col] = 1.0f / r.s;
        argmax[col] = r.a;
    }
    if (seed_B > 0) {
        for (int j = threadIdx.x; j < seed_B; j += 64) {
            seed_masked[j] = j != 0;
            if (j != 0) argmax[j] = 0;
        }
        if (threadIdx.x == 0) *gate_out = seed_B - 1;
    }
}

// One workgroup of 16 waves: wave w merges positions w, w + 16, ... exactly
// as lmhead_combine_kernel does, then wave 0 commits the block.
__global__ __launch_bounds__(1024) void lmhead_combine_commit_kernel(
    const void* __restrict__ ws, int G, int B, float* __restrict__ conf,
    int32_t* __restrict__ argmax, float tau, uint8_t* __restrict__ masked,
    int32_t* __restrict__ tokens, int32_t* __restrict__ n_committed, const int32_t* gate,
    int32_t* gate_out, int32_t* steps) {
    // gate and gate_out are the same word inside the block loop: the gate is
    // read here, before the commit below replaces it.
    if (gated_off(gate)) return;
    __shared__ float sconf[64];
    __shared__ int sarg[64];
    const WsView w = ws_view(const_cast<void*>(ws), G, B);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    // The masked flags are read now, with the partials, not after the merge
    // (every wave reads them, unconditionally, so no branch waits on them).
    const int mk = masked[min(lane, B - 1)];
    for (int col = wave; col < B; col += 16) {
        const ArgSoft r = reduce_column(w, G, col);
        if (lane == 0) {
            const float c = 1.0f / r.s;
            conf[col] = c;
            argmax[col] = r.a;
            sconf[col] = c;
            sarg[col] = r.a;
        }
    }
    __syncthreads();
    if (wave == 0)
        commit_wave_flag(lane < B && mk != 0, lane < B ? sconf[lane] : 0.f, lane < B ? sarg[lane] : 0, B,
                         tau, masked, tokens, n_committed, gate_out, steps);
}

}  // namespace

hipError_t launch_combine(void* ws, int G, int B, const Finish& f, hipStream_t st) {
    if (f.accept_draft != nullptr) {
        auto k = B <= 16 ? lmhead_combine_accept_kernel<64>
                         : (B <= 32 ? lmhead_combine_accept_kernel<32>
                                    : lmhead_combine_accept_kernel<16>);
        hipLaunchKernelGGL(k, dim3(1), dim3(1024), 0, st, ws, G, B, f.conf, f.argmax,
                           f.accept_draft, f.accept_B, f.accept_P, int(f.accept_bonus),
                           f.accepted, f.kv_len, f.out_tokens);
    } else if (f.commit)
        hipLaunchKernelGGL(lmhead_combine_commit_kernel, dim3(1), dim3(1024), 0, st, ws, G, B,
                           f.conf, f.argmax, f.tau, f.masked, f.tokens, f.n_committed, f.gate,
                           f.gate_out, f.steps);
    else
        hipLaunchKernelGGL(lmhead_combine_kernel, dim3(B), dim3(64), 0, st, ws, G, B, f.conf,
                           f.argmax, f.gate, f.seed_B, f.seed_masked, f.gate_out);
    return hipGetLastError();
}


namespace {

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  NB = number of 16-position column blocks (ceil(B/16));
// NCH = 128-element K chunks per wave.  blockDim.x = 64 * ks, d = 128*NCH*ks.
//
// Load path.  Wave w owns the K range [w*NCH*128, (w+1)*NCH*128) of every
// tile, i.e. a 16-row x NCH*256-byte region.  It reads that region with
// 4*NCH non-temporal 16-byte loads per lane, where consecutive lanes read
// consecutive 16-byte pieces (each instruction covers 1 KB of contiguous
// memory, whole cache lines; the weights are used once, so they bypass the
// caches), stages it in a wave-private LDS buffer and reads the MFMA A
// fragments from there.  Row r's 16-byte piece p sits in LDS slot p ^ (r % 16)
// of that row, so the 16 rows read by one fragment load fall in 16 distinct
// banks.  The next tile's loads are in flight while the current tile is
// multiplied.
// ---------------------------------------------------------------------------
template <int NB, int NCH, int KS = 4>
__global__ __launch_bounds__(64 * KS) void lmhead_bf16_kernel(const uint16_t* __restrict__ h,
                                                              const uint16_t* __restrict__ W,
                                                              int B, int d, int V, int ntiles,
                                                              void* __restrict__ ws,
                                                              const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    constexpr int NL = NCH * 4;                       // 16-byte loads per lane per tile
    constexpr int PIECES = NCH * 16;                  // 16-byte pieces per row segment
    __shared__ f32x4 red[2][KS][NB][64];              // per-wave partial logits, 2 buffers
    __shared__ ArgSoft fin[KS][NB][16];
    __shared__ __align__(16) u32x4 stage[KS][16 * PIECES];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int kw = wave * NCH * 128;                  // this wave's K start (elements)
    const int G = gridDim.x;

    // B fragments of h for this wave's K range, kept in registers: fragment
    // (c, j) of lane (r16, g) holds k = kw + 128c + 32g + 8j .. +7.
    bf16x8 hf[NCH][4][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = nb * 16 + r16;
        const u32x4* hp =
            reinterpret_cast<const u32x4*>(h + size_t(row < B ? row : 0) * d + kw + g * 32);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 v = (row < B) ? hp[c * 16 + j] : u32x4{0, 0, 0, 0};
                hf[c][j][nb] = __builtin_bit_cast(bf16x8, v);
            }
    }

    ArgSoft st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st[nb] = ArgSoft{-INFINITY, 0.f, 0x7fffffff};

    // Load i of a lane covers slot q = 64 i + lane of the row-major
    // [16 rows][PIECES] region: row q / PIECES, slot q % PIECES, holding
    // piece (slot ^ row % 16).
    auto load_tile = [&](u32x4 (&buf)[NL], int tile) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int q = 64 * i + lane;
            const int r = q / PIECES;
            const int piece = (q % PIECES) ^ (r & 15);
            int row = tile * 16 + r;
            row = row < V ? row : V - 1;
            buf[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(W + size_t(row) * d + kw) + piece);
        }
    };

    // Contiguous range of tiles per workgroup.
    const int t_beg = int(int64_t(ntiles) * blockIdx.x / G);
    const int t_end = int(int64_t(ntiles) * (blockIdx.x + 1) / G);
    u32x4 nxt[NL];
    if (t_beg < t_end) load_tile(nxt, t_beg);
    int it = 0;
    for (int tile = t_beg; tile < t_end; ++tile, ++it) {
        // The previous tile's fragment reads precede these writes in this
        // wave's program order, so the wave-private buffer can be refilled.
#pragma unroll
        for (int i = 0; i < NL; ++i) stage[wave][64 * i + lane] = nxt[i];
        if (tile + 1 < t_end) load_tile(nxt, tile + 1);

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int piece = c * 16 + g * 4 + j;
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, stage[wave][r16 * PIECES + (piece ^ r16)]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hf[c][j][nb], acc[nb],
                                                                      0, 0, 0);
            }

        if (nwave > 1) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) red[it & 1][wave][nb][lane] = acc[nb];
            __syncthreads();
        }
        // Position block nb of this tile is added up and folded by wave
        // (it + nb * nwave / NB) % nwave, so with several blocks different
        // waves fold them side by side.
        const int row0 = tile * 16 + g * 4;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int folder = (it + nb * (nwave >= NB ? nwave / NB : 1)) % nwave;
            if (wave == folder) {
                f32x4 t = acc[nb];
                if (nwave > 1) {
                    t = red[it & 1][0][nb][lane];
                    for (int w = 1; w < nwave; ++w) t += red[it & 1][w][nb][lane];
                }
                const float x[4] = {t[0] * kLog2e, t[1] * kLog2e, t[2] * kLog2e, t[3] * kLog2e};
                fold4(st[nb], x, row0, V);
            }
        }
    }

    store_workgroup_partials<NB>(st, fin, ws, B);
}

// Generic bf16 fallback for shapes whose h fragments do not fit in
// registers (large B x d): one wave per 16-row tile over the whole K range,
// h fragments re-read (from cache) per chunk.
template <int NB>
__global__ __launch_bounds__(256) void lmhead_bf16_generic_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int B, int d, int V,
    int ntiles, void* __restrict__ ws, const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    __shared__ ArgSoft fin[4][NB][16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int G = gridDim.x;

    ArgSoft st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st[nb] = ArgSoft{-INFINITY, 0.f, 0x7fffffff};

    for (int tile = blockIdx.x * nwave + wave; tile < ntiles; tile += G * nwave) {
        int row = tile * 16 + r16;
        row = row < V ? row : V - 1;
        const u32x4* wp = reinterpret_cast<const u32x4*>(W + size_t(row) * d + g * 32);
        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < d / 128; ++c) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, wp[c * 16 + j]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int hrow = nb * 16 + r16;
                    const u32x4* hp =
                        reinterpret_cast<const u32x4*>(h + size_t(hrow < B ? hrow : 0) * d + g * 32);
                    const u32x4 hv = (hrow < B) ? hp[c * 16 + j] : u32x4{0, 0, 0, 0};
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(bf16x8, hv), acc[nb], 0, 0, 0);
                }
            }
        }
        const int row0 = tile * 16 + g * 4;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float x[4] = {acc[nb][0] * kLog2e, acc[nb][1] * kLog2e, acc[nb][2] * kLog2e,
                                acc[nb][3] * kLog2e};
            fold4(st[nb], x, row0, V);
        }
    }
    store_workgroup_partials<NB>(st, fin, ws, B);
}

// ---------------------------------------------------------------------------
// float32 path (small problems): workgroup (x, b) scans vocabulary slice x
// for position b, one row per thread, h[b] staged in LDS.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 256;

__global__ __launch_bounds__(256) void lmhead_f32_kernel(const float* __restrict__ h,
                                                         const float* __restrict__ W, int B,
                                                         int d, int V, void* __restrict__ ws,
                                                         const int32_t* __restrict__ gate) {
    if (gated_off(gate)) return;
    extern __shared__ float hs[];
    __shared__ ArgSoft wst[4];
    const int b = blockIdx.y;
    for (int k = threadIdx.x; k < d; k += blockDim.x) hs[k] = h[size_t(b) * d + k];
    __syncthreads();
    const int v = blockIdx.x * kF32Rows + threadIdx.x;
    ArgSoft st{-INFINITY, 0.f, 0x7fffffff};
    if (v < V) {
        const float* wr = W + size_t(v) * d;
        float acc = 0.f;
        for (int k = 0; k < d; ++k) acc = fmaf(hs[k], wr[k], acc);
        st = ArgSoft{acc * kLog2e, 1.f, v};
    }
    for (int off = 1; off < 64; off <<= 1) st = merge(st, shfl_xor_state(st, off));
    if ((threadIdx.x & 63) == 0) wst[threadIdx.x >> 6] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgSoft s = wst[0];
        for (int w = 1; w < 4; ++w) s = merge(s, wst[w]);
        store_partial(ws_view(ws, gridDim.x, B), gridDim.x, b, blockIdx.x, s);
    }
}

// Host-side plan for the bf16 kernel: waves per workgroup (K split) and
// chunks per wave.  Returns false when the register-resident variant does not
// apply (then the generic kernel runs).
// Waves per workgroup (ks, splitting K) and 128-element chunks per wave
// (nch) of the streaming kernel: four waves when h's fragments fit, else
// eight with at most two chunks each (the LDS holds eight waves' stages only
// then), which covers 33 to 64 positions at d = 2048 (two waves per SIMD).
bool plan_bf16(int B, int d, int* ks, int* nch) {
    const int NB = (B + 15) / 16;
    const int c = d / 128;
    const int max_nch = 8 / NB;       // h fragments: 16 * NCH * NB VGPRs <= 128
    const int order[4] = {4, 2, 1, 8};
    for (int i = 0; i < 4; ++i) {
        const int k = order[i];
        if (k == 8 && c / k > 2) continue;
        if (c % k == 0 && c / k <= max_nch) {
            *ks = k;
            *nch = c / k;
            return true;
        }
    }
    return false;
}

template <int NB>
hipError_t launch_nb(const void* h, const void* W, int B, int d, int V, const Finish& f,
                     void* ws, hipStream_t st) {
    const int ntiles = (V + 15) / 16;
    const int G = lmhead_grid(B, d, V);
    const auto* hh = static_cast<const uint16_t*>(h);
    const auto* ww = static_cast<const uint16_t*>(W);
    int ks = 0, nch = 0;
    if (!plan_bf16(B, d, &ks, &nch)) {
        hipLaunchKernelGGL(lmhead_bf16_generic_kernel<NB>, dim3(G), dim3(256), 0, st, hh, ww, B,
                           d, V, ntiles, ws, f.gate);
        const hipError_t e = hipGetLastError();
        return e != hipSuccess ? e : launch_combine(ws, G, B, f, st);
    }
#define BD_LMH_CASE(N)                                                                     \
    case N:                                                                                \
        if constexpr (N * NB > 8) {                                                        \
            return hipErrorInvalidValue;                                                   \
        } else if constexpr (N <= 2) {                                                     \
            if (ks == 8)                                                                   \
                hipLaunchKernelGGL((lmhead_bf16_kernel<NB, N, 8>), dim3(G), dim3(512), 0,  \
                                   st, hh, ww, B, d, V, ntiles, ws, f.gate);               \
            else                                                                           \
                hipLaunchKernelGGL((lmhead_bf16_kernel<NB, N>), dim3(G), dim3(64 * ks), 0, \
                                   st, hh, ww, B, d, V, ntiles, ws, f.gate);               \
        } else {                                                                           \
            hipLaunchKernelGGL((lmhead_bf16_kernel<NB, N>), dim3(G), dim3(64 * ks), 0, st, \
                               hh, ww, B, d, V, ntiles, ws, f.gate);                       \
        }                                                                                  \
        break;
    switch (nch) {
        BD_LMH_CASE(1)
        BD_LMH_CASE(2)
        BD_LMH_CASE(3)
        BD_LMH_CASE(4)
        BD_LMH_CASE(5)
        BD_LMH_CASE(6)
        BD_LMH_CASE(7)
        BD_LMH_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef BD_LMH_CASE
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine(ws, G, B, f, st);
}

}  // namespace

int lmhead_grid(int B, int d, int V) {
    (void)B;
    (void)d;
    return persistent_grid((V + 15) / 16);
}

size_t lmhead_ws_bytes_dt(bd_dtype dt, int B, int d, int V) {
    // bf16: one partial per workgroup and position; f32: one per 256-row
    // vocabulary slice and position.
    const int G = dt == BD_F32 ? (V + kF32Rows - 1) / kF32Rows : lmhead_grid(B, d, V);
    return ws_size(G, B);
}

size_t lmhead_ws_bytes(int B, int d, int V) {
    const size_t a = lmhead_ws_bytes_dt(BD_BF16, B, d, V);
    const size_t b = lmhead_ws_bytes_dt(BD_F32, B, d, V);
    return a > b ? a : b;
}

hipError_t launch_lmhead_bf16(const void* h, const void* W, int B, int d, int V, const Finish& f,
                              void* ws, hipStream_t st) {
    switch ((B + 15) / 16) {
        case 1: return launch_nb<1>(h, W, B, d, V, f, ws, st);
        case 2: return launch_nb<2>(h, W, B, d, V, f, ws, st);
        case 3: return launch_nb<3>(h, W, B, d, V, f, ws, st);
        case 4: return launch_nb<4>(h, W, B, d, V, f, ws, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lmhead_f32(const float* h, const float* W, int B, int d, int V,
                             const Finish& f, void* ws, hipStream_t st) {
    const dim3 grid((V + kF32Rows - 1) / kF32Rows, B);
    hipLaunchKernelGGL(lmhead_f32_kernel, grid, dim3(kF32Rows), size_t(d) * sizeof(float), st, h,
                       W, B, d, V, ws, f.gate);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_combine(ws, grid.x, B, f, st);
}

}  // namespace bd
