/*
 * ep_probe.h -- measurement kernels (libep_probe.so), not part of the method.
 *
 * Each probe moves the same bytes as one of libep.so's operations in the
 * simplest pattern there is, so that a benchmark can report an operation's
 * rate beside a ceiling measured on the same GPU in the same run:
 *   ep_probe_write      only the packed rows' stores (16-byte nontemporal)
 *   ep_probe_pack       read each token row once, store it to n_t "planes"
 *                       (the dispatch's bytes, with no segment scatter)
 *   ep_probe_reduce     read n_t planes per token, add in fp32, store one bf16
 *                       row (the combine's bytes and arithmetic, no gather)
 *   ep_probe_empty      an empty kernel of a given grid (launch floor)
 *   ep_probe_ll_copy    the low-latency dispatch's copy with its grid, cells
 *                       known in advance (no slot computation)
 *   ep_probe_ll_reduce  the low-latency combine's loads, weighted fp32 sum and
 *                       store, cells known in advance
 * Conventions are those of ep.h: device pointers, 16-byte aligned rows,
 * hidden % 8 == 0, stream-ordered, no host synchronization.  Every call
 * returns an ep_status; arguments out of range give EP_ERR_INVALID and
 * misaligned pointers EP_ERR_ALIGN before anything is enqueued.
 */
#ifndef EP_PROBE_H
#define EP_PROBE_H

#include <stdint.h>

#include "ep.h"

#ifdef __cplusplus
extern "C" {
#endif

/* bytes (a multiple of 16) of dst written with 16-byte nontemporal stores. */
int ep_probe_write(void *dst, int64_t bytes, ep_stream_t stream);

/* x [T][hidden] bf16; rows_per_token [T] int32 in [0, kmax];
 * planes [kmax][T][hidden] bf16: planes[j][t] = x[t] for j < rows_per_token[t]
 * (nontemporal stores, 128 lanes per token like the pack). */
int ep_probe_pack(const void *x, int32_t T, int32_t hidden, const int32_t *rows_per_token,
                  int32_t kmax, void *planes, ep_stream_t stream);

/* out[t] = bf16_rne(sum over j < rows_per_token[t] of fp32(planes[j][t])),
 * nontemporal loads and stores, 128 lanes per token like the combine. */
int ep_probe_reduce(const void *planes, int32_t T, int32_t hidden, const int32_t *rows_per_token,
                    int32_t kmax, void *out, ep_stream_t stream);

/* An empty kernel of `blocks` workgroups of `threads` (64..1024) threads. */
int ep_probe_empty(int32_t blocks, int32_t threads, ep_stream_t stream);

/* cells [T*K][hidden] bf16: cells[t*K + k] = x[t] for every k, with the
 * low-latency dispatch's grid (workgroups of 512 threads, one slice of about
 * 512 vectors of one token each); plain stores like that dispatch. */
int ep_probe_ll_copy(const void *x, int32_t T, int32_t hidden, int32_t K, void *cells,
                     ep_stream_t stream);

/* out[t] = bf16_rne(sum over k of w[t][k] * fp32(cells[t*K + k])) with fp32
 * fma in ascending k, the low-latency combine's grid (workgroups of 256
 * threads, one 16-byte vector each). */
int ep_probe_ll_reduce(const void *cells, const float *w, int32_t T, int32_t hidden, int32_t K,
                       void *out, ep_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_PROBE_H */
