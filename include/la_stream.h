/*
 * la_stream.h — C ABI of libla_stream.so: streaming kernels that measure the
 * HBM bandwidth the GPU reaches in practice, the reference the benchmark sets
 * beside the published 8 TB/s peak.  Not part of the attention path.
 *
 * la_stream_run: one launch over src_bytes of device memory at src (rounded
 * down to whole 64 KiB steps of a 256-thread workgroup; 60 KiB for mode 2),
 * with `grid` workgroups walking the steps grid-stride, on `stream`
 * (a hipStream_t, NULL for the default stream).
 *   mode 0  read src only; each thread of each workgroup writes one word of
 *           what it read to sink[workgroup * 256 + thread] (sink holds
 *           grid * 256 unsigned), so no load is dead.
 *   mode 1  copy: dst = src (dst at least src_bytes).
 *   mode 2  read + write 3:2, the byte mix of the forward output kernel (q,
 *           k, v read, o written): per step 15 vectors read, 10 written;
 *           dst holds 2/3 of the source's bytes.
 *   mode 3  in-place update: every 16-byte vector of src is read, changed
 *           and written back to the same address (the decode step's access
 *           pattern on its states); dst is unused.
 *   nontemporal  1: streaming (non-temporal) loads and stores.
 * Returns 0, 1 for invalid arguments (nothing launched), 2 for a launch error.
 * Pointers must be 16-byte aligned device memory owned by the caller.
 *
 * la_stream_bytes_moved: bytes one la_stream_run call reads plus writes
 * (0 for an unknown mode).
 */
#ifndef LIGHTNING_LA_STREAM_H
#define LIGHTNING_LA_STREAM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int la_stream_run(int mode, int nontemporal, const void* src, void* dst, size_t src_bytes, unsigned* sink,
                  int grid, void* stream);
size_t la_stream_bytes_moved(int mode, size_t src_bytes);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_LA_STREAM_H */
