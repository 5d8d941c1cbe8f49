/*
 * bdiff_probe.h - measurement reference of libbdiff (not a step of the
 * method).  The decode step is bound by HBM bandwidth (Fast-dVLM overview
 * §1.1: batch-1 decoding reloads every weight per step), so its kernels are
 * reported against the chip's published peak and against what a plain
 * streaming read of a large buffer achieves on the same GPU.
 * Conventions as in bdiff.h.
 */
#ifndef BDIFF_PROBE_H
#define BDIFF_PROBE_H

#include "bdiff.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bd_probe_stream_read - reads n_bytes of src once, with `grid` workgroups of
 * 256 threads (one contiguous chunk per workgroup, 8 non-temporal 16-byte
 * loads in flight per thread), and XOR-accumulates the data into *sink:
 *   *sink ^= XOR over every 32-bit word of src[0 .. n_bytes)
 * (so the caller may check it; zero *sink first for the plain checksum).
 *   src   device buffer, 16-byte aligned;  sink  device uint32, 4-byte aligned
 * Limits: n_bytes > 0 and a multiple of 16; 1 <= grid <= 65536.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_LAUNCH.
 */
bd_status bd_probe_stream_read(const void* src, size_t n_bytes, int32_t grid, uint32_t* sink,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BDIFF_PROBE_H */
