// Internal declarations shared by the libbdiff translation units: vector
// types for gfx950 MFMA operands, small device helpers, and the kernel
// launchers that the C ABI layer calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdiff.h"

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// bfloat16 bits -> float32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two packed bfloat16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Gate of a step of the device-resident block loop: the number of block
// positions still masked, written by the previous step's commit.  A kernel
// given a gate that reads 0 returns at once (the block is complete); a null
// gate always runs.
__device__ __forceinline__ bool gated_off(const int32_t* gate) {
    return gate != nullptr && *gate == 0;
}

// Softmax partial state (max in log2 units, sum of 2^(x - max), index).
struct ArgSoft {
    float m;
    float s;
    int a;
};

// Merge two partial states: larger max wins the index, equal maxima keep the
// smaller index, sums are rescaled to the common max.
__device__ __forceinline__ ArgSoft merge(ArgSoft x, ArgSoft y) {
    if (y.m > x.m || (y.m == x.m && y.a < x.a)) {
        ArgSoft t = x;
        x = y;
        y = t;
    }
    // x now holds the winner
    if (y.s > 0.f) x.s += y.s * exp2f(y.m - x.m);
    return x;
}

// Kernel launchers (defined next to their kernels).  They assume validated
// arguments and return the HIP launch status.
hipError_t launch_commit(const float* conf, const int32_t* argmax, int B, float tau,
                         uint8_t* masked, int32_t* tokens, int32_t* n_committed, hipStream_t st);
hipError_t launch_spec_accept(const int32_t* draft, const int32_t* verify, int B, int P,
                              int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                              hipStream_t st, bool bonus = false);
hipError_t launch_cert_scan(const float* conf, const int32_t* atok, const int32_t* ttok, int n,
                            int k, int32_t* order, int32_t* accepted, int32_t* skip,
                            hipStream_t st);
// Start of the device-resident block loop: gate = masked positions, the step
// counter and the per-step commit counts zeroed.
hipError_t launch_loop_init(const uint8_t* masked, int B, int32_t* gate, int32_t* steps,
                            int32_t* n_committed, int S, hipStream_t st);
// Start of a block of the multi-block loop (one workgroup): kv_len advances
// by `advance` (clamped to [0, len_max]); with `append`, the block's K/V rows
// k_new, v_new ([B][Hkv][128] bf16) are written into cache rows kv_len ..
// kv_len + B - 1; steps and n_committed[0 .. S) (if given) are zeroed and
// *zero_word (if given) cleared.
hipError_t launch_block_begin(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              int cap, int Hkv, int B, int32_t* kv_len, int advance, int len_max,
                              bool append, int32_t* steps, int32_t* n_committed, int S,
                              uint64_t* zero_word, hipStream_t st);

// LM head.  The merge of the per-workgroup partials writes conf/argmax and,
// when `commit` is set, also applies the threshold commit to the block.
struct Finish {
    float* conf;
    int32_t* argmax;
    bool commit;
    float tau;
    uint8_t* masked;
    int32_t* tokens;
    int32_t* n_committed;
    // Device-resident block loop only (null otherwise): the step's gate (see
    // gated_off), where the commit leaves the next gate (the same word), and
    // the executed-step counter it increments.
    const int32_t* gate = nullptr;
    int32_t* gate_out = nullptr;
    int32_t* steps = nullptr;
    // AR seed of a block (multi-block loop; 0 otherwise): the merge of a
    // one-row LM head writes the seed token through `argmax` (pointing at the
    // block's tokens: position 0), token 0 at positions 1 .. seed_B - 1, marks
    // those masked and position 0 committed in seed_masked, and sets
    // *gate_out to seed_B - 1.
    int seed_B = 0;
    uint8_t* seed_masked = nullptr;
    // Speculative accept after the merge (null accept_draft otherwise): the
    // verify tokens are this call's argmax at positions 0 .. accept_B - 1,
    // compared with accept_draft[0 .. accept_B) as bd_spec_accept(_bonus) does.
    const int32_t* accept_draft = nullptr;
    int accept_B = 0;
    int accept_P = 0;
    bool accept_bonus = false;
    int32_t* accepted = nullptr;
    int32_t* kv_len = nullptr;
    int32_t* out_tokens = nullptr;
};
int lmhead_grid(int B, int d, int V);           // workgroups used for a shape
size_t lmhead_ws_bytes(int B, int d, int V);              // either dtype
size_t lmhead_ws_bytes_dt(bd_dtype dt, int B, int d, int V);
hipError_t launch_lmhead_bf16(const void* h, const void* W, int B, int d, int V, const Finish& f,
                              void* ws, hipStream_t st);
hipError_t launch_lmhead_f32(const float* h, const float* W, int B, int d, int V,
                             const Finish& f, void* ws, hipStream_t st);
// Host checks of an LM-head call's arguments (everything but the workspace),
// and the launch of the dt path on a validated workspace.
bd_status lmhead_args_status(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                             int32_t V, const Finish& f);
hipError_t launch_lmhead(bd_dtype dt, const void* h, const void* W, int B, int d, int V,
                         const Finish& f, void* ws, hipStream_t st);

// FP8 (E4M3, W8A8) LM head and the per-row quantizer it applies to h.
int lmhead_fp8_grid(int B, int d, int V);
size_t lmhead_fp8_ws_bytes(int B, int d, int V);
hipError_t launch_lmhead_fp8(const void* h, const uint8_t* W, const float* w_scale, int B, int d,
                             int V, const Finish& f, void* ws, hipStream_t st);
hipError_t launch_quant_fp8_rows(const void* x, int R, int d, uint8_t* q, float* scale,
                                 hipStream_t st);

// Block attention.  P_dev (nullable): a device-side prefix length, at most P,
// read by the kernels in place of P (the grid and workspace are sized for P).
size_t block_attn_ws_bytes(int P, int Bq, int Hq, int Hkv, int dh);
hipError_t launch_block_attn_bf16(const void* q, const void* kc, const void* vc, int P, int cap,
                                  const uint64_t* mask, int Bq, int Hq, int Hkv, float scale,
                                  void* out, void* ws, hipStream_t st,
                                  const int32_t* gate = nullptr,
                                  const int32_t* P_dev = nullptr);
// Paged cache: pools [n_pages][Hkv][page_size][128], logical keys from key_lo.
hipError_t launch_block_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* page_table, int page_size, int n_pages, int P,
                                   int key_lo, const uint64_t* mask, int Bq, int Hq, int Hkv,
                                   float scale, void* out, void* ws, hipStream_t st);
// FP8 (E4M3) KV cache: codes [Hkv][cap][128], per-KV-head float32 scales.
hipError_t launch_block_attn_fp8kv(const void* q, const uint8_t* kc, const uint8_t* vc,
                                   const float* k_scale, const float* v_scale, int P, int cap,
                                   const uint64_t* mask, int Bq, int Hq, int Hkv, float scale,
                                   void* out, void* ws, hipStream_t st);
// New rows x [n][Hkv][dh] (bf16) into cache rows pos .. pos+n-1 of an FP8 cache.
hipError_t launch_kv_quant_fp8(const void* x, int n, int Hkv, int dh, const float* scale,
                               uint8_t* cache, int cap, int pos, hipStream_t st);
hipError_t launch_block_attn_f32(const float* q, const float* kc, const float* vc, int P, int cap,
                                 const uint64_t* mask, int Bq, int Hq, int Hkv, int dh,
                                 float scale, float* out, hipStream_t st,
                                 const int32_t* gate = nullptr);

// Dual-stream attention.  seg (host, n_seg entries) holds the text segment
// starts of the auto-truncation mask; null means one segment.
constexpr int kMaxSegments = 64;
// lse (nullable): the row log-sum-exp [N][H] (natural log) for the backward.
hipError_t launch_dualstream_bf16(const void* q, const void* k, const void* v, int n_vis,
                                  int n_txt, int block, int H, float scale, void* out,
                                  hipStream_t st, const int32_t* seg = nullptr, int n_seg = 1,
                                  float* lse = nullptr);
hipError_t launch_dualstream_f32(const float* q, const float* k, const float* v, int n_vis,
                                 int n_txt, int block, int H, int dh, float scale, float* out,
                                 hipStream_t st, const int32_t* seg = nullptr, int n_seg = 1,
                                 float* lse = nullptr);
// Backward: dq, dk, dv from q, k, v, out, d_out and the forward's lse; ws
// holds D = rowsum(d_out * out) [N][H] float.
size_t dualstream_bwd_ws_bytes(int N, int H);
hipError_t launch_dualstream_bwd_bf16(const void* q, const void* k, const void* v,
                                      const void* out, const void* dout, const float* lse,
                                      int n_vis, int n_txt, int block, const int32_t* seg,
                                      int n_seg, int H, float scale, void* dq, void* dk, void* dv,
                                      void* ws, hipStream_t st);
hipError_t launch_dualstream_bwd_f32(const float* q, const float* k, const float* v,
                                     const float* out, const float* dout, const float* lse,
                                     int n_vis, int n_txt, int block, const int32_t* seg,
                                     int n_seg, int H, int dh, float scale, float* dq, float* dk,
                                     float* dv, void* ws, hipStream_t st);

}  // namespace bd
