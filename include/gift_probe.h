/*
 * gift_probe.h -- HBM streaming probes (libgift_probe.so).
 *
 * Measurement tools, not part of the GIFT path: each call launches one
 * kernel that streams a device buffer in one access pattern, so that the
 * caller can time it with events on the same stream.  They give the ceiling
 * of the access patterns the round-trip kernels use (a plain or
 * nontemporal float4 stream; the 64 x 256 tiles of the quantize and
 * un-whiten passes, read in one load round; the 64-row slabs of the whiten
 * pass, walked 32 columns at a time by 8 waves).
 *
 * Arguments are device pointers (16-byte aligned) and sizes in bytes or
 * elements; `stream` is a hipStream_t (NULL = the null stream).  The buffers
 * are read or written, never allocated or freed.  Return: 0 on success, 1 for
 * a bad argument (NULL or misaligned pointer, size not a multiple of 16
 * bytes, matrix shape not a multiple of the pattern), 4 if the launch
 * failed.  Read probes leave memory unchanged.
 */
#ifndef GIFT_PROBE_H
#define GIFT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* read `bytes` of buf as float4 (nontemporal loads if nontemporal != 0) */
int gift_probe_read(const void* buf, size_t bytes, int nontemporal, void* stream);
/* write `bytes` of buf as float4 zeros */
int gift_probe_write(void* buf, size_t bytes, int nontemporal, void* stream);
/* copy `bytes` from src to dst as float4 */
int gift_probe_copy(const void* src, void* dst, size_t bytes, int nontemporal, void* stream);
/* read a row-major fp32 matrix (rows % 64 == 0, cols % 256 == 0) in
 * 64 x 256 tiles, one workgroup of 8 waves per tile, each lane loading its
 * 16-row MFMA fragments' float4s in one round */
int gift_probe_tile_read(const float* m, int64_t rows, int64_t cols, void* stream);
/* write zeros to the same matrix in 64 x 256 tiles, each lane storing the
 * float4s of its 16-row MFMA fragments (16 rows x 64 bytes per store
 * instruction) */
int gift_probe_tile_write(float* m, int64_t rows, int64_t cols, int nontemporal, void* stream);
/* read the same matrix in 64-row slabs (rows % 64 == 0, cols % 256 == 0),
 * one workgroup of 8 waves per slab, wave w walking the 32-column chunks
 * w, w + 8, ... with the next chunk's loads in flight */
int gift_probe_slab_read(const float* m, int64_t rows, int64_t cols, void* stream);

#ifdef __cplusplus
}
#endif

#endif
