// Threshold commit of one block, executed by one full wavefront (lane i owns
// position i, B <= 64).  Shared by the standalone commit kernel and the
// LM-head merge kernel that commits right after it.
#pragma once

#include "bd_internal.h"

namespace bd {

// Every masked position with conf > tau is committed; if none qualifies and
// some position is masked, the most confident masked position (lowest index
// on ties) is committed alone.  Committing sets tokens[i] = argmax and
// masked[i] = 0.  Must be called by all 64 lanes of a wave; c/a are lane i's
// confidence and token (ignored for i >= B).  Inside the device-resident
// block loop (else both null), `gate_out` receives the number of positions
// still masked afterwards (the next step's gate) and `steps` counts the step.
// `was_masked` is lane i's masked[i] != 0 (false for i >= B), read by the
// caller, which can then issue that read early.
__device__ __forceinline__ void commit_wave_flag(bool was_masked, float c, int32_t a, int B,
                                                 float tau, uint8_t* __restrict__ masked,
                                                 int32_t* __restrict__ tokens,
                                                 int32_t* __restrict__ n_committed,
                                                 int32_t* gate_out, int32_t* steps) {
    const int i = threadIdx.x & 63;
    const bool m = was_masked;
    const bool above = m && (c > tau);
    const uint64_t above_bits = __ballot(above);
    const uint64_t masked_bits = __ballot(m);
    bool take = above;
    int n = __popcll(above_bits);
    if (above_bits == 0 && masked_bits != 0) {
        float bc = c;
        int bi = m ? i : 64;
        for (int off = 32; off > 0; off >>= 1) {
            const float oc = __shfl_xor(bc, off);
            const int oi = __shfl_xor(bi, off);
            const bool other_valid = oi < 64;
            const bool mine_valid = bi < 64;
            if (other_valid && (!mine_valid || oc > bc || (oc == bc && oi < bi))) {
                bc = oc;
                bi = oi;
            }
        }
        take = (i == bi);
        n = 1;
    }
    if (take) {
        tokens[i] = a;
        masked[i] = 0;
    }
    if (i == 0) {
        *n_committed = n;
        if (gate_out != nullptr) *gate_out = __popcll(masked_bits) - n;
        if (steps != nullptr) *steps += 1;
    }
}

// Longest verified prefix (Fast-dVLM overview §2.3.1), executed by one full
// wavefront: lane i holds draft token d and verify token v of position i
// (ignored for i >= B).  The first disagreement is the lowest set bit of a
// ballot.  out_tokens[0 .. L) = draft, accepted = L and kv_len = P + L; with
// `bonus` the verify token at the first disagreement is appended too
// (accepted = L + 1 when L < B), the cache still keeping P + L rows.  Shared
// by the standalone accept kernel and the LM-head merge that accepts right
// after it.
__device__ __forceinline__ void accept_wave(bool bonus, int32_t d, int32_t v, int B, int P,
                                            int32_t* __restrict__ accepted,
                                            int32_t* __restrict__ kv_len,
                                            int32_t* __restrict__ out_tokens) {
    const int i = threadIdx.x & 63;
    const bool differ = i < B && d != v;
    const uint64_t bits = __ballot(differ);
    const int L = bits ? __builtin_ctzll(bits) : B;
    if (i < L) out_tokens[i] = d;
    if (bonus && i == L && L < B) out_tokens[i] = v;
    if (i == 0) {
        *accepted = bonus && L < B ? L + 1 : L;
        *kv_len = P + L;
    }
}

__device__ __forceinline__ void commit_wave(float c, int32_t a, int B, float tau,
                                            uint8_t* __restrict__ masked,
                                            int32_t* __restrict__ tokens,
                                            int32_t* __restrict__ n_committed,
                                            int32_t* gate_out = nullptr,
                                            int32_t* steps = nullptr) {
    const int i = threadIdx.x & 63;
    commit_wave_flag(i < B && masked[i] != 0, c, a, B, tau, masked, tokens, n_committed,
                     gate_out, steps);
}

}  // namespace bd
