// C ABI of libbdiff: argument validation on the host, then the kernel
// launchers.  Nothing is enqueued unless every check passes; no call touches
// the HIP runtime before its arguments are validated, so the error paths run
// (and are tested) on machines without a GPU.
#include <math.h>
#include <string.h>

#include "bd_internal.h"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bd_status launch_status(hipError_t e) { return e == hipSuccess ? BD_OK : BD_E_LAUNCH; }

inline float default_scale(float scale, int dh) {
    return scale != 0.f ? scale : 1.0f / sqrtf(static_cast<float>(dh));
}

// Vocabulary sizes up to 2^30 (tile counts stay far inside int32).
inline bool vocab_ok(int32_t V) { return V >= 1 && V <= (1 << 30); }

bool dh_ok(bd_dtype dt, int dh) {
    if (dt == BD_BF16) return dh == 128;
    return dh >= 4 && dh <= 128 && dh % 4 == 0;
}

}  // namespace

extern "C" {

const char* bd_status_str(bd_status s) {
    switch (s) {
        case BD_OK: return "ok";
        case BD_E_NULL: return "a required pointer is NULL";
        case BD_E_SHAPE: return "size out of range or inconsistent sizes";
        case BD_E_DTYPE: return "unsupported dtype for this call";
        case BD_E_ALIGN: return "pointer not 16-byte aligned";
        case BD_E_WORKSPACE: return "workspace missing or too small";
        case BD_E_DEVICE: return "device is not gfx950";
        case BD_E_LAUNCH: return "kernel launch failed";
        default: break;
    }
    return "unknown status";
}

bd_status bd_device_check(int device) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
        return BD_E_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return BD_E_DEVICE;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? BD_OK : BD_E_DEVICE;
}

bd_status bd_make_intra_mask(bd_mask_kind kind, int32_t Bq, uint64_t* host_rows) {
    if (!host_rows) return BD_E_NULL;
    if (Bq < 1 || Bq > 64) return BD_E_SHAPE;
    if (kind == BD_MASK_SPEC_FUSED && (Bq & 1)) return BD_E_SHAPE;
    const uint64_t ones = (Bq == 64) ? ~0ull : ((1ull << Bq) - 1ull);
    for (int i = 0; i < Bq; ++i) {
        uint64_t row = 0;
        switch (kind) {
            case BD_MASK_BIDIR: row = ones; break;
            case BD_MASK_CAUSAL: row = (i == 63) ? ~0ull : ((1ull << (i + 1)) - 1ull); break;
            case BD_MASK_SPEC_FUSED: {
                const int B = Bq / 2;
                const uint64_t half = (1ull << B) - 1ull;
                if (i < B) {
                    row = (1ull << (i + 1)) - 1ull;                  // verify half: causal
                } else {
                    const int r = i - B;
                    row = ((1ull << (r + 1)) - 1ull) | (half << B);   // j <= i-B, all drafts
                }
                break;
            }
            default: return BD_E_SHAPE;
        }
        host_rows[i] = row;
    }
    return BD_OK;
}

size_t bd_block_attn_ws_bytes(int32_t P, int32_t Bq, int32_t Hq, int32_t Hkv, int32_t dh) {
    if (P < 0 || Bq < 1 || Bq > 64 || Hq < 1 || Hkv < 1 || dh < 1) return 0;
    return bd::block_attn_ws_bytes(P, Bq, Hq, Hkv, dh);
}

bd_status bd_block_attn(bd_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                        int32_t P, int32_t cap, const uint64_t* intra_mask, int32_t Bq,
                        int32_t Hq, int32_t Hkv, int32_t dh, float scale, void* out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !intra_mask || !out) return BD_E_NULL;
    if (dt != BD_F32 && dt != BD_BF16) return BD_E_DTYPE;
    if (Bq < 1 || Bq > 64 || P < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return BD_E_SHAPE;
    if ((int64_t)P + Bq > cap) return BD_E_SHAPE;
    if (!dh_ok(dt, dh)) return BD_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return BD_E_ALIGN;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    const float sc = default_scale(scale, dh);
    if (dt == BD_F32)
        return launch_status(bd::launch_block_attn_f32(
            static_cast<const float*>(q), static_cast<const float*>(k_cache),
            static_cast<const float*>(v_cache), P, cap, intra_mask, Bq, Hq, Hkv, dh, sc,
            static_cast<float*>(out), stream));
    if ((int64_t)P + Bq > 65536) return BD_E_SHAPE;   // at most 1024 key tiles
    const size_t need = bd::block_attn_ws_bytes(P, Bq, Hq, Hkv, dh);
    if (!ws || ws_bytes < need) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    return launch_status(bd::launch_block_attn_bf16(q, k_cache, v_cache, P, cap, intra_mask, Bq,
                                                    Hq, Hkv, sc, out, ws, stream));
}

bd_status bd_block_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* page_table, int32_t page_size, int32_t n_pages,
                              int32_t P, int32_t key_lo, const uint64_t* intra_mask, int32_t Bq,
                              int32_t Hq, int32_t Hkv, int32_t dh, float scale, void* out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k_pool || !v_pool || !page_table || !intra_mask || !out) return BD_E_NULL;
    if (Bq < 1 || Bq > 64 || P < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return BD_E_SHAPE;
    if (dh != 128 || page_size < 1 || n_pages < 1 || key_lo < 0 || key_lo > P) return BD_E_SHAPE;
    const int64_t n_keys = (int64_t)P + Bq;
    if (n_keys - key_lo > 65536) return BD_E_SHAPE;              // at most 1024 key tiles
    if ((n_keys + page_size - 1) / page_size > n_pages) return BD_E_SHAPE;
    if ((int64_t)n_pages * Hkv * page_size * dh * 2 >= ((int64_t)1 << 32)) return BD_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
        return BD_E_ALIGN;
    const size_t need = bd::block_attn_ws_bytes(P - key_lo, Bq, Hq, Hkv, dh);
    if (!ws || ws_bytes < need) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    return launch_status(bd::launch_block_attn_paged(q, k_pool, v_pool, page_table, page_size,
                                                     n_pages, P, key_lo, intra_mask, Bq, Hq, Hkv,
                                                     default_scale(scale, dh), out, ws, stream));
}

bd_status bd_block_attn_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                              const float* k_scale, const float* v_scale, int32_t P, int32_t cap,
                              const uint64_t* intra_mask, int32_t Bq, int32_t Hq, int32_t Hkv,
                              int32_t dh, float scale, void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !intra_mask || !out)
        return BD_E_NULL;
    if (Bq < 1 || Bq > 64 || P < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return BD_E_SHAPE;
    if ((int64_t)P + Bq > cap || (int64_t)P + Bq > 65536 || dh != 128) return BD_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return BD_E_ALIGN;
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u)
        return BD_E_ALIGN;
    const size_t need = bd::block_attn_ws_bytes(P, Bq, Hq, Hkv, dh);
    if (!ws || ws_bytes < need) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    return launch_status(bd::launch_block_attn_fp8kv(q, k_cache, v_cache, k_scale, v_scale, P,
                                                     cap, intra_mask, Bq, Hq, Hkv,
                                                     default_scale(scale, dh), out, ws, stream));
}

bd_status bd_kv_quant_fp8(const void* x, int32_t n, int32_t Hkv, int32_t dh, const float* scale,
                          uint8_t* cache, int32_t cap, int32_t pos, hipStream_t stream) {
    if (!x || !scale || !cache) return BD_E_NULL;
    if (n < 0 || Hkv < 1 || dh < 4 || dh % 4 != 0 || pos < 0 || cap < 1) return BD_E_SHAPE;
    if ((int64_t)pos + n > cap) return BD_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(x) & 7u) || (reinterpret_cast<uintptr_t>(cache) & 3u) ||
        (reinterpret_cast<uintptr_t>(scale) & 3u))
        return BD_E_ALIGN;
    return launch_status(bd::launch_kv_quant_fp8(x, n, Hkv, dh, scale, cache, cap, pos, stream));
}

size_t bd_lmhead_conf_ws_bytes(int32_t B, int32_t d, int32_t V) {
    if (B < 1 || B > 64 || d < 1 || !vocab_ok(V)) return 0;
    return bd::lmhead_ws_bytes(B, d, V);
}

}  // extern "C"

namespace bd {

bd_status lmhead_args_status(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                             int32_t V, const Finish& f) {
    if (!h || !W || !f.conf || !f.argmax) return BD_E_NULL;
    if (f.commit && (!f.masked || !f.tokens || !f.n_committed)) return BD_E_NULL;
    if (dt != BD_F32 && dt != BD_BF16) return BD_E_DTYPE;
    if (B < 1 || B > 64 || d < 1 || !vocab_ok(V)) return BD_E_SHAPE;
    if (dt == BD_BF16 && (d % 128 != 0 || d > 16384)) return BD_E_SHAPE;
    if (f.commit && !(f.tau == f.tau)) return BD_E_SHAPE;
    if (!aligned16(h) || !aligned16(W)) return BD_E_ALIGN;
    return BD_OK;
}

hipError_t launch_lmhead(bd_dtype dt, const void* h, const void* W, int B, int d, int V,
                         const Finish& f, void* ws, hipStream_t st) {
    if (dt == BD_F32)
        return launch_lmhead_f32(static_cast<const float*>(h), static_cast<const float*>(W), B, d,
                                 V, f, ws, st);
    return launch_lmhead_bf16(h, W, B, d, V, f, ws, st);
}

}  // namespace bd

extern "C" {

namespace {

bd_status lmhead_common(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                        int32_t V, const bd::Finish& f, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
    const bd_status s = bd::lmhead_args_status(dt, h, W, B, d, V, f);
    if (s != BD_OK) return s;
    if (!ws || ws_bytes < bd::lmhead_ws_bytes(B, d, V)) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    return launch_status(bd::launch_lmhead(dt, h, W, B, d, V, f, ws, stream));
}

}  // namespace

bd_status bd_lmhead_conf(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                         int32_t V, float* conf, int32_t* argmax, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    const bd::Finish f{conf, argmax, false, 0.f, nullptr, nullptr, nullptr};
    return lmhead_common(dt, h, W, B, d, V, f, ws, ws_bytes, stream);
}

bd_status bd_lmhead_conf_commit(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                                int32_t V, float tau, float* conf, int32_t* argmax,
                                uint8_t* masked, int32_t* tokens, int32_t* n_committed, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    const bd::Finish f{conf, argmax, true, tau, masked, tokens, n_committed};
    return lmhead_common(dt, h, W, B, d, V, f, ws, ws_bytes, stream);
}

bd_status bd_lmhead_conf_accept(bd_dtype dt, const void* h, const void* W, int32_t B, int32_t d,
                                int32_t V, float* conf, int32_t* argmax, const int32_t* draft,
                                int32_t B_acc, int32_t P, int32_t bonus, int32_t* accepted,
                                int32_t* kv_len, int32_t* out_tokens, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
    if (!draft || !accepted || !kv_len || !out_tokens) return BD_E_NULL;
    bd::Finish f{conf, argmax, false, 0.f, nullptr, nullptr, nullptr};
    const bd_status s = bd::lmhead_args_status(dt, h, W, B, d, V, f);
    if (s != BD_OK) return s;
    if (B_acc < 1 || B_acc > B || P < 0 || (int64_t)P + B_acc > INT32_MAX) return BD_E_SHAPE;
    f.accept_draft = draft;
    f.accept_B = B_acc;
    f.accept_P = P;
    f.accept_bonus = bonus != 0;
    f.accepted = accepted;
    f.kv_len = kv_len;
    f.out_tokens = out_tokens;
    return lmhead_common(dt, h, W, B, d, V, f, ws, ws_bytes, stream);
}

size_t bd_lmhead_conf_fp8_ws_bytes(int32_t B, int32_t d, int32_t V) {
    if (B < 1 || B > 64 || d < 128 || d > 16384 || d % 128 != 0 || !vocab_ok(V)) return 0;
    return bd::lmhead_fp8_ws_bytes(B, d, V);
}

namespace {

bd_status lmhead_fp8_common(const void* h, const uint8_t* Wq, const float* w_scale, int32_t B,
                            int32_t d, int32_t V, const bd::Finish& f, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    if (!h || !Wq || !w_scale || !f.conf || !f.argmax) return BD_E_NULL;
    if (f.commit && (!f.masked || !f.tokens || !f.n_committed)) return BD_E_NULL;
    if (B < 1 || B > 64 || !vocab_ok(V) || d < 128 || d > 16384 || d % 128 != 0) return BD_E_SHAPE;
    if (f.commit && !(f.tau == f.tau)) return BD_E_SHAPE;
    if (!aligned16(h) || !aligned16(Wq) || !aligned16(w_scale)) return BD_E_ALIGN;
    if (!ws || ws_bytes < bd::lmhead_fp8_ws_bytes(B, d, V)) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    return launch_status(bd::launch_lmhead_fp8(h, Wq, w_scale, B, d, V, f, ws, stream));
}

}  // namespace

bd_status bd_lmhead_conf_fp8(const void* h, const uint8_t* Wq, const float* w_scale, int32_t B,
                             int32_t d, int32_t V, float* conf, int32_t* argmax, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    const bd::Finish f{conf, argmax, false, 0.f, nullptr, nullptr, nullptr};
    return lmhead_fp8_common(h, Wq, w_scale, B, d, V, f, ws, ws_bytes, stream);
}

bd_status bd_lmhead_conf_commit_fp8(const void* h, const uint8_t* Wq, const float* w_scale,
                                    int32_t B, int32_t d, int32_t V, float tau, float* conf,
                                    int32_t* argmax, uint8_t* masked, int32_t* tokens,
                                    int32_t* n_committed, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    const bd::Finish f{conf, argmax, true, tau, masked, tokens, n_committed};
    return lmhead_fp8_common(h, Wq, w_scale, B, d, V, f, ws, ws_bytes, stream);
}

bd_status bd_quant_fp8_rows(const void* x, int32_t R, int32_t d, uint8_t* q, float* scale,
                            hipStream_t stream) {
    if (!x || !q || !scale) return BD_E_NULL;
    if (R < 0 || d < 8 || d % 8 != 0) return BD_E_SHAPE;
    if (!aligned16(x) || !aligned16(q)) return BD_E_ALIGN;
    return launch_status(bd::launch_quant_fp8_rows(x, R, d, q, scale, stream));
}

namespace {

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct LoopWs {
    size_t attn_off, lm_off, total;
};

LoopWs loop_ws(int32_t P, int32_t B, int32_t Hq, int32_t Hkv, int32_t dh, int32_t d, int32_t V,
               bool fp8) {
    LoopWs L;
    L.attn_off = 256;                                       // the gate word
    L.lm_off = L.attn_off + al256(bd::block_attn_ws_bytes(P, B, Hq, Hkv, dh));
    L.total = L.lm_off + al256(fp8 ? bd::lmhead_fp8_ws_bytes(B, d, V)
                                   : bd::lmhead_ws_bytes(B, d, V));
    return L;
}

}  // namespace

size_t bd_block_loop_ws_bytes(int32_t P, int32_t B, int32_t Hq, int32_t Hkv, int32_t dh,
                              int32_t d, int32_t V, int32_t w_fp8) {
    if (P < 0 || B < 1 || B > 64 || Hq < 1 || Hkv < 1 || dh < 1 || d < 1 || !vocab_ok(V)) return 0;
    if (w_fp8 && (d < 128 || d > 16384 || d % 128 != 0)) return 0;
    return loop_ws(P, B, Hq, Hkv, dh, d, V, w_fp8 != 0).total;
}

bd_status bd_block_loop(bd_dtype dt, const void* q_steps, const void* k_cache,
                        const void* v_cache, int32_t P, int32_t cap, const uint64_t* intra_mask,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                        const void* h_steps, const void* W, const float* w_scale, int32_t d,
                        int32_t V, float tau, int32_t max_steps, uint8_t* masked,
                        int32_t* tokens, void* attn_out, float* conf, int32_t* argmax,
                        int32_t* n_committed, int32_t* n_steps, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
    if (!q_steps || !k_cache || !v_cache || !intra_mask || !h_steps || !W || !masked ||
        !tokens || !attn_out || !conf || !argmax || !n_committed || !n_steps)
        return BD_E_NULL;
    if (dt != BD_F32 && dt != BD_BF16) return BD_E_DTYPE;
    const bool fp8 = w_scale != nullptr;
    if (fp8 && dt != BD_BF16) return BD_E_DTYPE;
    // attention limits (bd_block_attn)
    if (B < 1 || B > 64 || P < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return BD_E_SHAPE;
    if ((int64_t)P + B > cap) return BD_E_SHAPE;
    if (!dh_ok(dt, dh)) return BD_E_SHAPE;
    if (dt == BD_BF16 && (int64_t)P + B > 65536) return BD_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    // LM-head limits (bd_lmhead_conf / bd_lmhead_conf_fp8)
    if (d < 1 || !vocab_ok(V)) return BD_E_SHAPE;
    if ((dt == BD_BF16 || fp8) && (d % 128 != 0 || d > 16384)) return BD_E_SHAPE;
    if (!(tau == tau)) return BD_E_SHAPE;
    if (max_steps < 1 || max_steps > 1024) return BD_E_SHAPE;
    if (!aligned16(q_steps) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(attn_out) || !aligned16(h_steps) || !aligned16(W) ||
        (fp8 && !aligned16(w_scale)))
        return BD_E_ALIGN;
    const LoopWs L = loop_ws(P, B, Hq, Hkv, dh, d, V, fp8);
    if (!ws || ws_bytes < L.total) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;

    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* gate = reinterpret_cast<int32_t*>(base);
    void* attn_ws = base + L.attn_off;
    void* lm_ws = base + L.lm_off;
    const float sc = default_scale(scale, dh);
    const size_t es = dt == BD_BF16 ? 2 : 4;
    const size_t q_step = size_t(B) * Hq * dh * es;
    const size_t h_step = size_t(B) * d * es;
    hipError_t e = bd::launch_loop_init(masked, B, gate, n_steps, n_committed, max_steps, stream);
    for (int s = 0; s < max_steps && e == hipSuccess; ++s) {
        const uint8_t* qs = static_cast<const uint8_t*>(q_steps) + s * q_step;
        uint8_t* os = static_cast<uint8_t*>(attn_out) + s * q_step;
        const uint8_t* hs = static_cast<const uint8_t*>(h_steps) + s * h_step;
        if (dt == BD_BF16)
            e = bd::launch_block_attn_bf16(qs, k_cache, v_cache, P, cap, intra_mask, B, Hq, Hkv,
                                           sc, os, attn_ws, stream, gate);
        else
            e = bd::launch_block_attn_f32(reinterpret_cast<const float*>(qs),
                                          static_cast<const float*>(k_cache),
                                          static_cast<const float*>(v_cache), P, cap, intra_mask,
                                          B, Hq, Hkv, dh, sc, reinterpret_cast<float*>(os),
                                          stream, gate);
        if (e != hipSuccess) break;
        bd::Finish f{conf + size_t(s) * B, argmax + size_t(s) * B, true, tau, masked, tokens,
                     n_committed + s};
        f.gate = gate;
        f.gate_out = gate;
        f.steps = n_steps;
        if (fp8)
            e = bd::launch_lmhead_fp8(hs, static_cast<const uint8_t*>(W), w_scale, B, d, V, f,
                                      lm_ws, stream);
        else if (dt == BD_BF16)
            e = bd::launch_lmhead_bf16(hs, W, B, d, V, f, lm_ws, stream);
        else
            e = bd::launch_lmhead_f32(reinterpret_cast<const float*>(hs),
                                      static_cast<const float*>(W), B, d, V, f, lm_ws, stream);
    }
    return launch_status(e);
}

namespace {

struct BlocksWs {
    size_t mask_off, attn_off, lm_off, total;
};

// Gate word at 0, the all-zero intra-block mask of the seed queries at 8,
// then one attention workspace (large enough for the last block's steps and
// every seed) and one LM-head workspace (B rows; the seed uses one).
BlocksWs blocks_ws(int32_t P_max, int32_t n_blocks, int32_t B, int32_t Hq, int32_t Hkv,
                   int32_t dh, int32_t d, int32_t V, bool fp8) {
    BlocksWs L;
    L.mask_off = 8;
    L.attn_off = 256;
    const int32_t P_last = P_max + (n_blocks - 1) * B;
    const size_t a1 = bd::block_attn_ws_bytes(P_last, B, Hq, Hkv, dh);
    const size_t a2 = bd::block_attn_ws_bytes(P_last, 1, Hq, Hkv, dh);
    L.lm_off = L.attn_off + al256(a1 > a2 ? a1 : a2);
    const size_t l1 = fp8 ? bd::lmhead_fp8_ws_bytes(B, d, V) : bd::lmhead_ws_bytes(B, d, V);
    const size_t l2 = fp8 ? bd::lmhead_fp8_ws_bytes(1, d, V) : bd::lmhead_ws_bytes(1, d, V);
    L.total = L.lm_off + al256(l1 > l2 ? l1 : l2);
    return L;
}

bool blocks_shape_ok(int32_t P_max, int32_t cap, int32_t n_blocks, int32_t B, int32_t Hq,
                     int32_t Hkv, int32_t dh, int32_t d, int32_t V) {
    if (n_blocks < 1 || B < 1 || B > 64 || P_max < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
        return false;
    if (dh != 128 || d < 128 || d > 16384 || d % 128 != 0 || !vocab_ok(V)) return false;
    const int64_t end = (int64_t)P_max + (int64_t)n_blocks * B;
    return end <= cap && end <= 65536;
}

}  // namespace

size_t bd_decode_blocks_ws_bytes(int32_t P_max, int32_t n_blocks, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t dh, int32_t d, int32_t V, int32_t w_fp8) {
    if (!blocks_shape_ok(P_max, 1 << 30, n_blocks, B, Hq, Hkv, dh, d, V)) return 0;
    return blocks_ws(P_max, n_blocks, B, Hq, Hkv, dh, d, V, w_fp8 != 0).total;
}

bd_status bd_decode_blocks(const void* q_seed, const void* h_seed, const void* q_steps,
                           const void* h_steps, const void* k_blk, const void* v_blk,
                           void* k_cache, void* v_cache, int32_t cap, int32_t* kv_len,
                           int32_t P_max, const uint64_t* intra_mask, int32_t n_blocks, int32_t B,
                           int32_t max_steps, int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                           const void* W, const float* w_scale, int32_t d, int32_t V, float tau,
                           int32_t* tokens, uint8_t* masked, int32_t* n_steps,
                           int32_t* n_committed, void* seed_attn, float* seed_conf,
                           void* attn_out, float* conf, int32_t* argmax, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
    if (!q_seed || !h_seed || !q_steps || !h_steps || !k_blk || !v_blk || !k_cache ||
        !v_cache || !kv_len || !intra_mask || !W || !tokens || !masked || !n_steps ||
        !n_committed || !seed_attn || !seed_conf || !attn_out || !conf || !argmax)
        return BD_E_NULL;
    const bool fp8 = w_scale != nullptr;
    if (!blocks_shape_ok(P_max, cap, n_blocks, B, Hq, Hkv, dh, d, V)) return BD_E_SHAPE;
    if (max_steps < 1 || max_steps > 1024) return BD_E_SHAPE;
    if (!(tau == tau)) return BD_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    if (!aligned16(q_seed) || !aligned16(h_seed) || !aligned16(q_steps) || !aligned16(h_steps) ||
        !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(W) || !aligned16(seed_attn) || !aligned16(attn_out) ||
        (fp8 && !aligned16(w_scale)) || (reinterpret_cast<uintptr_t>(kv_len) & 3u))
        return BD_E_ALIGN;
    const BlocksWs L = blocks_ws(P_max, n_blocks, B, Hq, Hkv, dh, d, V, fp8);
    if (!ws || ws_bytes < L.total) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;

    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* gate = reinterpret_cast<int32_t*>(base);
    uint64_t* zero_mask = reinterpret_cast<uint64_t*>(base + L.mask_off);
    void* attn_ws = base + L.attn_off;
    void* lm_ws = base + L.lm_off;
    const float sc = default_scale(scale, dh);
    const size_t row_q = size_t(Hq) * dh * 2;             // one query row, bf16
    const size_t row_h = size_t(d) * 2;
    const size_t blk_kv = size_t(B) * Hkv * dh * 2;
    const size_t step_q = size_t(B) * row_q, step_h = size_t(B) * row_h;
    auto lm = [&](const void* h, int rows, const bd::Finish& f) {
        return fp8 ? bd::launch_lmhead_fp8(h, static_cast<const uint8_t*>(W), w_scale, rows, d,
                                           V, f, lm_ws, stream)
                   : bd::launch_lmhead_bf16(h, W, rows, d, V, f, lm_ws, stream);
    };
    hipError_t e = hipSuccess;
    for (int b = 0; b < n_blocks && e == hipSuccess; ++b) {
        const int P_b = P_max + b * B;                    // bound of this block's prefix
        int32_t* tok_b = tokens + size_t(b) * B;
        uint8_t* msk_b = masked + size_t(b) * B;
        int32_t* ncom_b = n_committed + size_t(b) * max_steps;
        // 1. the previous block joins the prefix; this block's rows go in
        e = bd::launch_block_begin(static_cast<const uint8_t*>(k_blk) + b * blk_kv,
                                   static_cast<const uint8_t*>(v_blk) + b * blk_kv, k_cache,
                                   v_cache, cap, Hkv, B, kv_len, b > 0 ? B : 0, P_b, true,
                                   n_steps + b, ncom_b, max_steps, zero_mask, stream);
        if (e != hipSuccess) break;
        // 2. AR seed: one query over the prefix, the LM head's argmax starts the block
        e = bd::launch_block_attn_bf16(static_cast<const uint8_t*>(q_seed) + b * row_q, k_cache,
                                       v_cache, P_b, cap, zero_mask, 1, Hq, Hkv, sc,
                                       static_cast<uint8_t*>(seed_attn) + b * row_q, attn_ws,
                                       stream, nullptr, kv_len);
        if (e != hipSuccess) break;
        bd::Finish fs{seed_conf + b, tok_b, false, 0.f, nullptr, nullptr, nullptr};
        fs.gate_out = gate;
        fs.seed_B = B;
        fs.seed_masked = msk_b;
        e = lm(static_cast<const uint8_t*>(h_seed) + b * row_h, 1, fs);
        // 3. denoising steps, each gated on the positions still masked
        for (int s = 0; s < max_steps && e == hipSuccess; ++s) {
            const size_t bs = size_t(b) * max_steps + s;
            e = bd::launch_block_attn_bf16(static_cast<const uint8_t*>(q_steps) + bs * step_q,
                                           k_cache, v_cache, P_b, cap, intra_mask, B, Hq, Hkv,
                                           sc, static_cast<uint8_t*>(attn_out) + bs * step_q,
                                           attn_ws, stream, gate, kv_len);
            if (e != hipSuccess) break;
            bd::Finish f{conf + bs * B, argmax + bs * B, true, tau, msk_b, tok_b, ncom_b + s};
            f.gate = gate;
            f.gate_out = gate;
            f.steps = n_steps + b;
            e = lm(static_cast<const uint8_t*>(h_steps) + bs * step_h, B, f);
        }
    }
    // 4. the last block joins the prefix
    if (e == hipSuccess)
        e = bd::launch_block_begin(nullptr, nullptr, k_cache, v_cache, cap, Hkv, B, kv_len, B,
                                   P_max + n_blocks * B, false, nullptr, nullptr, 0, nullptr,
                                   stream);
    return launch_status(e);
}

bd_status bd_commit(const float* conf, const int32_t* argmax, int32_t B, float tau,
                    uint8_t* masked, int32_t* tokens, int32_t* n_committed, hipStream_t stream) {
    if (!conf || !argmax || !masked || !tokens || !n_committed) return BD_E_NULL;
    if (B < 0 || B > 64) return BD_E_SHAPE;
    if (!(tau == tau)) return BD_E_SHAPE;
    return launch_status(bd::launch_commit(conf, argmax, B, tau, masked, tokens, n_committed,
                                           stream));
}

bd_status bd_spec_accept(const int32_t* draft, const int32_t* verify, int32_t B, int32_t P,
                         int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                         hipStream_t stream) {
    if (!draft || !verify || !accepted || !kv_len || !out_tokens) return BD_E_NULL;
    if (B < 0 || B > 64 || P < 0 || (int64_t)P + B > INT32_MAX) return BD_E_SHAPE;
    return launch_status(
        bd::launch_spec_accept(draft, verify, B, P, accepted, kv_len, out_tokens, stream));
}

bd_status bd_spec_accept_bonus(const int32_t* draft, const int32_t* verify, int32_t B, int32_t P,
                               int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                               hipStream_t stream) {
    if (!draft || !verify || !accepted || !kv_len || !out_tokens) return BD_E_NULL;
    if (B < 0 || B > 64 || P < 0 || (int64_t)P + B > INT32_MAX) return BD_E_SHAPE;
    return launch_status(bd::launch_spec_accept(draft, verify, B, P, accepted, kv_len, out_tokens,
                                                stream, true));
}

bd_status bd_cert_scan(const float* anchor_conf, const int32_t* anchor_tok,
                       const int32_t* text_tok, int32_t n, int32_t k, int32_t* order,
                       int32_t* accepted, int32_t* skip_full, hipStream_t stream) {
    if (!anchor_conf || !anchor_tok || !text_tok || !order || !accepted || !skip_full)
        return BD_E_NULL;
    if (n < 0 || n > 1024) return BD_E_SHAPE;
    return launch_status(bd::launch_cert_scan(anchor_conf, anchor_tok, text_tok, n, k, order,
                                              accepted, skip_full, stream));
}

namespace {

// Checks of a segmentation given as a host array (null = one segment).
bd_status check_segments(const int32_t* seg, int32_t n_seg, int32_t n_txt) {
    if (!seg) return BD_OK;
    if (n_seg < 1 || n_seg > bd::kMaxSegments || seg[0] != 0) return BD_E_SHAPE;
    for (int s = 1; s < n_seg; ++s)
        if (seg[s] <= seg[s - 1] || seg[s] >= n_txt) return BD_E_SHAPE;
    return BD_OK;
}

// Shape, dtype and alignment checks shared by the dual-stream calls.
bd_status dualstream_check(bd_dtype dt, int32_t n_vis, int32_t n_txt, int32_t block, int32_t H,
                           int32_t dh, float scale) {
    if (dt != BD_F32 && dt != BD_BF16) return BD_E_DTYPE;
    if (n_vis < 0 || n_txt < 0 || block < 1 || H < 1) return BD_E_SHAPE;
    const int64_t N = (int64_t)n_vis + 2 * (int64_t)n_txt;
    if (N < 1 || N > (1 << 24)) return BD_E_SHAPE;
    if (!dh_ok(dt, dh)) return BD_E_SHAPE;
    if (!(scale >= 0.f) || isinf(scale)) return BD_E_SHAPE;
    return BD_OK;
}

bd_status dualstream_common(bd_dtype dt, const void* q, const void* k, const void* v,
                            int32_t n_vis, int32_t n_txt, int32_t block, const int32_t* seg,
                            int32_t n_seg, int32_t H, int32_t dh, float scale, void* out,
                            hipStream_t stream, float* lse = nullptr) {
    if (!q || !k || !v || !out) return BD_E_NULL;
    const bd_status s = dualstream_check(dt, n_vis, n_txt, block, H, dh, scale);
    if (s != BD_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return BD_E_ALIGN;
    const float sc = default_scale(scale, dh);
    if (dt == BD_F32)
        return launch_status(bd::launch_dualstream_f32(
            static_cast<const float*>(q), static_cast<const float*>(k),
            static_cast<const float*>(v), n_vis, n_txt, block, H, dh, sc,
            static_cast<float*>(out), stream, seg, n_seg, lse));
    return launch_status(bd::launch_dualstream_bf16(q, k, v, n_vis, n_txt, block, H, sc, out,
                                                    stream, seg, n_seg, lse));
}

}  // namespace

bd_status bd_dualstream_attn(bd_dtype dt, const void* q, const void* k, const void* v,
                             int32_t n_vis, int32_t n_txt, int32_t block, int32_t H, int32_t dh,
                             float scale, void* out, hipStream_t stream) {
    return dualstream_common(dt, q, k, v, n_vis, n_txt, block, nullptr, 1, H, dh, scale, out,
                             stream);
}

bd_status bd_dualstream_attn_seg(bd_dtype dt, const void* q, const void* k, const void* v,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H,
                                 int32_t dh, float scale, void* out, hipStream_t stream) {
    if (!seg_starts) return BD_E_NULL;
    const bd_status s = check_segments(seg_starts, n_seg, n_txt);
    if (s != BD_OK) return s;
    return dualstream_common(dt, q, k, v, n_vis, n_txt, block, seg_starts, n_seg, H, dh, scale,
                             out, stream);
}

bd_status bd_dualstream_attn_fwd(bd_dtype dt, const void* q, const void* k, const void* v,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H,
                                 int32_t dh, float scale, void* out, float* lse,
                                 hipStream_t stream) {
    const bd_status s = check_segments(seg_starts, n_seg, n_txt);
    if (s != BD_OK) return s;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return BD_E_ALIGN;
    return dualstream_common(dt, q, k, v, n_vis, n_txt, block, seg_starts,
                             seg_starts ? n_seg : 1, H, dh, scale, out, stream, lse);
}

size_t bd_dualstream_attn_bwd_ws_bytes(int32_t n_vis, int32_t n_txt, int32_t H) {
    const int64_t N = (int64_t)n_vis + 2 * (int64_t)n_txt;
    if (n_vis < 0 || n_txt < 0 || H < 1 || N < 1 || N > (1 << 24)) return 0;
    return bd::dualstream_bwd_ws_bytes(int(N), H);
}

bd_status bd_dualstream_attn_bwd(bd_dtype dt, const void* q, const void* k, const void* v,
                                 const void* out, const void* d_out, const float* lse,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H, int32_t dh,
                                 float scale, void* dq, void* dk, void* dv, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !out || !d_out || !lse || !dq || !dk || !dv) return BD_E_NULL;
    bd_status s = dualstream_check(dt, n_vis, n_txt, block, H, dh, scale);
    if (s != BD_OK) return s;
    s = check_segments(seg_starts, n_seg, n_txt);
    if (s != BD_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(d_out) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return BD_E_ALIGN;
    const int N = n_vis + 2 * n_txt;
    if (!ws || ws_bytes < bd::dualstream_bwd_ws_bytes(N, H)) return BD_E_WORKSPACE;
    if (!aligned16(ws)) return BD_E_ALIGN;
    const float sc = default_scale(scale, dh);
    const int ns = seg_starts ? n_seg : 1;
    if (dt == BD_F32)
        return launch_status(bd::launch_dualstream_bwd_f32(
            static_cast<const float*>(q), static_cast<const float*>(k),
            static_cast<const float*>(v), static_cast<const float*>(out),
            static_cast<const float*>(d_out), lse, n_vis, n_txt, block, seg_starts, ns, H, dh, sc,
            static_cast<float*>(dq), static_cast<float*>(dk), static_cast<float*>(dv), ws,
            stream));
    return launch_status(bd::launch_dualstream_bwd_bf16(q, k, v, out, d_out, lse, n_vis, n_txt,
                                                        block, seg_starts, ns, H, sc, dq, dk, dv,
                                                        ws, stream));
}

}  // extern "C"
