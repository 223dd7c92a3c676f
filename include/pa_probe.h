/*
 * libpa_probe -- bandwidth reference points for the attention kernels.
 *
 * Measurement only: these kernels read device memory and compute nothing the
 * attention path needs.  They give the denominators of "% of achievable":
 *
 *   pa_probe_stream_read  a plain streaming read of one large buffer (the
 *                         best the chip's HBM delivers to a read-only kernel);
 *   pa_probe_tile_read    the decode's own reads -- for every (piece, KV head,
 *                         sequence) the first L_b rows of each cache block the
 *                         block table names, K then V, in the decode's grid
 *                         order -- with no arithmetic on them, so the time is
 *                         what that access pattern alone costs.
 *
 * Both return PA_PROBE_OK (0) or a negative status; the message of the last
 * failure on the calling thread is pa_probe_last_error().  Pointers are
 * device pointers; stream is a hipStream_t (NULL = default stream).  Neither
 * call allocates or synchronises.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PA_PROBE_OK = 0, PA_PROBE_ERR_INVALID_ARG = -1, PA_PROBE_ERR_HIP = -4 };

const char* pa_probe_last_error(void);

/*
 * Read bytes (a positive multiple of 16, buf 16-byte aligned) once with
 * 16-byte non-temporal loads.  grid = number of 256-thread workgroups
 * (0 = 4096); each thread keeps four loads in flight.  sink: one uint32_t,
 * written only when the XOR of everything read equals a fixed constant (so
 * the loads cannot be dropped; the value itself is meaningless).
 */
int pa_probe_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream);

/*
 * The decode's read pattern over a head-major paged cache
 * [kv_heads, num_blocks, 16, row_bytes / elem]: one workgroup of `waves`
 * waves (4 or 8) per (piece, KV head, sequence), ids in piece-major order; a
 * piece covers split_tokens positions (a multiple of 16); wave w reads tiles
 * w, w + waves, ...; each tile is the first min(16, L_b - 16 j) rows of the
 * block named by block_tables[b, j], K then V.  row_bytes is 128 or 256
 * (one 16-byte chunk per lane per row group), block size 16.  Table entries
 * outside [0, num_blocks) are skipped.  sink as above.
 */
int pa_probe_tile_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int num_seqs, int kv_heads,
                       int max_blocks_per_seq, int num_blocks, int row_bytes, int split_tokens,
                       int max_context_len, int waves, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
