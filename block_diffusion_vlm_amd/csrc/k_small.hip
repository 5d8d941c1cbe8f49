// Latency-bound decisions of the decode step: threshold commit, speculative
// accept and the LOWN certificate scan.  Each runs in a single workgroup; a
// block holds at most 64 positions, so commit and accept are one wavefront
// with ballots instead of loops.
#include "commit_impl.h"

namespace bd {

// Threshold unmasking with the always-one rule (Fast-dVLM overview §4.1:
// denoising threshold 0.9).  Lane i owns position i.
__global__ __launch_bounds__(64) void commit_kernel(const float* __restrict__ conf,
                                                    const int32_t* __restrict__ argmax, int B,
                                                    float tau, uint8_t* __restrict__ masked,
                                                    int32_t* __restrict__ tokens,
                                                    int32_t* __restrict__ n_committed) {
    const int i = threadIdx.x;
    const float c = i < B ? conf[i] : 0.f;
    const int32_t a = i < B ? argmax[i] : 0;
    commit_wave(c, a, B, tau, masked, tokens, n_committed);
}

// Longest verified prefix (overview §2.3.1; accept_wave).  With BONUS the
// verify token at the first disagreement is appended too (greedy speculative
// decoding's correction token); the cache keeps P + L rows either way.
template <bool BONUS>
__global__ __launch_bounds__(64) void spec_accept_kernel(const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ verify,
                                                         int B, int P,
                                                         int32_t* __restrict__ accepted,
                                                         int32_t* __restrict__ kv_len,
                                                         int32_t* __restrict__ out_tokens) {
    const int i = threadIdx.x;
    const int32_t d = i < B ? draft[i] : 0;
    const int32_t v = i < B ? verify[i] : 0;
    accept_wave(BONUS, d, v, B, P, accepted, kv_len, out_tokens);
}

// LOWN certificate (method step details (2)-(3)).  Thread i computes the
// rank of position i in the stable descending order of anchor confidence;
// the certified prefix ends at the smallest rank whose text-only token
// disagrees with the anchor token, so no explicit sort is needed for L.
__global__ __launch_bounds__(1024) void cert_scan_kernel(const float* __restrict__ conf,
                                                         const int32_t* __restrict__ atok,
                                                         const int32_t* __restrict__ ttok, int n,
                                                         int k, int32_t* __restrict__ order,
                                                         int32_t* __restrict__ accepted,
                                                         int32_t* __restrict__ skip) {
    __shared__ float sc[1024];
    __shared__ int wave_min[16];
    const int i = threadIdx.x;
    if (i < n) sc[i] = conf[i];
    __syncthreads();
    int first_bad = n;
    if (i < n) {
        const float c = sc[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) {
            const float o = sc[j];
            rank += (o > c) || (o == c && j < i);
        }
        order[rank] = i;
        if (ttok[i] != atok[i]) first_bad = rank;
    }
    for (int off = 32; off > 0; off >>= 1) first_bad = min(first_bad, __shfl_xor(first_bad, off));
    if ((i & 63) == 0) wave_min[i >> 6] = first_bad;
    __syncthreads();
    if (i == 0) {
        int L = n;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) L = min(L, wave_min[w]);
        *accepted = L;
        *skip = (L >= k) ? 1 : 0;
    }
}

// Start of the device-resident block loop (one wave): the gate is the number
// of masked positions, the step counter and the per-step commit counts start
// at zero.
__global__ __launch_bounds__(64) void loop_init_kernel(const uint8_t* __restrict__ masked, int B,
                                                       int32_t* __restrict__ gate,
                                                       int32_t* __restrict__ steps,
                                                       int32_t* __restrict__ n_committed, int S) {
    const int i = threadIdx.x;
    const uint64_t bits = __ballot(i < B && masked[i] != 0);
    for (int s = i; s < S; s += 64) n_committed[s] = 0;
    if (i == 0) {
        *gate = __popcll(bits);
        *steps = 0;
    }
}

// Start of a block of the multi-block loop (overview §1.2: the earlier
// blocks stay in the KV cache; §2.2.2: the block's rows join it): one
// workgroup; every thread reads the old length before thread 0 stores the
// new one.
__global__ __launch_bounds__(256) void block_begin_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int cap, int Hkv, int B, int32_t* __restrict__ kv_len,
    int advance, int len_max, int append, int32_t* __restrict__ steps,
    int32_t* __restrict__ n_committed, int S, uint64_t* __restrict__ zero_word) {
    const int len = max(0, min(*kv_len + advance, len_max));
    if (append) {
        // 16 pieces of 16 bytes per 128-element row; row i of head g
        for (int p = threadIdx.x; p < B * Hkv * 16; p += blockDim.x) {
            const int piece = p & 15;
            const int ig = p >> 4;                  // i * Hkv + g
            const int g = ig % Hkv;
            const int i = ig / Hkv;
            const size_t dst = (size_t(g) * cap + len + i) * 16 + piece;
            k_cache[dst] = k_new[size_t(ig) * 16 + piece];
            v_cache[dst] = v_new[size_t(ig) * 16 + piece];
        }
    }
    for (int s = threadIdx.x; s < S; s += blockDim.x) n_committed[s] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        *kv_len = len;
        if (steps != nullptr) *steps = 0;
        if (zero_word != nullptr) *zero_word = 0;
    }
}

hipError_t launch_block_begin(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              int cap, int Hkv, int B, int32_t* kv_len, int advance, int len_max,
                              bool append, int32_t* steps, int32_t* n_committed, int S,
                              uint64_t* zero_word, hipStream_t st) {
    hipLaunchKernelGGL(block_begin_kernel, dim3(1), dim3(256), 0, st,
                       static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), cap, Hkv, B,
                       kv_len, advance, len_max, append ? 1 : 0, steps, n_committed, S,
                       zero_word);
    return hipGetLastError();
}

hipError_t launch_loop_init(const uint8_t* masked, int B, int32_t* gate, int32_t* steps,
                            int32_t* n_committed, int S, hipStream_t st) {
    hipLaunchKernelGGL(loop_init_kernel, dim3(1), dim3(64), 0, st, masked, B, gate, steps,
                       n_committed, S);
    return hipGetLastError();
}

hipError_t launch_commit(const float* conf, const int32_t* argmax, int B, float tau,
                         uint8_t* masked, int32_t* tokens, int32_t* n_committed, hipStream_t st) {
    hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, st, conf, argmax, B, tau, masked,
                       tokens, n_committed);
    return hipGetLastError();
}

hipError_t launch_spec_accept(const int32_t* draft, const int32_t* verify, int B, int P,
                              int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                              hipStream_t st, bool bonus) {
    if (bonus)
        hipLaunchKernelGGL(spec_accept_kernel<true>, dim3(1), dim3(64), 0, st, draft, verify, B,
                           P, accepted, kv_len, out_tokens);
    else
        hipLaunchKernelGGL(spec_accept_kernel<false>, dim3(1), dim3(64), 0, st, draft, verify, B,
                           P, accepted, kv_len, out_tokens);
    return hipGetLastError();
}

hipError_t launch_cert_scan(const float* conf, const int32_t* atok, const int32_t* ttok, int n,
                            int k, int32_t* order, int32_t* accepted, int32_t* skip,
                            hipStream_t st) {
    const int threads = n <= 64 ? 64 : ((n + 63) / 64) * 64;
    hipLaunchKernelGGL(cert_scan_kernel, dim3(1), dim3(threads), 0, st, conf, atok, ttok, n, k,
                       order, accepted, skip);
    return hipGetLastError();
}

}  // namespace bd
