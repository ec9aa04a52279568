/*
 * dsa_roofline.h -- ceiling probes of the benchmark (libdsa_roofline.so).
 *
 * These kernels are not part of the attention path.  They measure, on the
 * GPU and in the run that times the path, the rates its kernels are compared
 * with: streaming HBM read and copy, back-to-back BF16 MFMA, and random
 * 256-byte row gathers.  Pointers are caller-owned device memory (16-byte
 * aligned); calls only enqueue on `stream` (a hipStream_t as void*; NULL is
 * the null stream).  Return 0 on success, 1 if the launch failed, 2 for an
 * invalid argument (nothing launched).  `sink` is a device word the kernels
 * may write so that their loads and products are not optimised away.
 */
#ifndef DSA_ROOFLINE_H
#define DSA_ROOFLINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) from src with 16-byte loads. */
int dsa_roofline_read(const void* src, size_t bytes, void* sink, void* stream);

/* Writes every byte of dst[0..bytes) (16-byte aligned, bytes % 16 == 0) with
 * 16-byte non-temporal stores, one per thread, in address order: the
 * streaming-write ceiling.  bytes / 4096 < 2^31. */
int dsa_roofline_write(void* dst, size_t bytes, void* stream);

/* Copies `bytes` (a multiple of 16) from src to dst with 16-byte loads and stores. */
int dsa_roofline_copy(const void* src, void* dst, size_t bytes, void* stream);

/* `workgroups` x 4 waves, each running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 on register operands; dsa_roofline_mfma_flops
 * gives the flops one launch performs. */
int dsa_roofline_mfma(void* sink, int workgroups, int iters, void* stream);
double dsa_roofline_mfma_flops(int workgroups, int iters);

/* Gathers rows[0..n_rows) (each an index of a 256-byte row of buf, < buf_bytes / 256), 16 lanes
 * per row with 16-byte loads: n_rows * 256 bytes read. */
int dsa_roofline_gather(const void* buf, size_t buf_bytes, const int32_t* rows, int n_rows,
                        void* sink, void* stream);

/* The K/V reads of a sparse-attention launch with 256-byte rows (D * element
 * size = 256) and nothing else: caches [B, L_cap, H_kv, 256 bytes], indices
 * [rows, k] (row r of sequence r / S; entries outside [0, L_cap) skipped).
 * Each wave reads the K and V rows of its 32-key tiles a 128-byte line per 8
 * lanes, two tiles in flight, at two 4-wave workgroups per CU.  wave_rows = 0:
 * one workgroup per (row, KV head), wave w reading tiles w, w + 4, ...;
 * wave_rows = 1: workgroup j takes KV head j % H_kv and rows 4 (j / H_kv) +
 * wave, each wave reading all tiles of its row in order (the two schedules
 * of the attention kernel).  rows, H_kv <= 65535. */
int dsa_roofline_kv_gather(const void* k_cache, const void* v_cache, const int32_t* indices,
                           int rows, int k, int S, int H_kv, int L_cap, int wave_rows, void* sink,
                           void* stream);

/* `workgroups` x `threads` (<= 1024) threads; every workgroup reads word[0]
 * and stores nothing (sink is only written for word[0] == 0x1234567): the
 * cost of launching a kernel that waits on one memory read. */
int dsa_roofline_floor(const int32_t* word, void* sink, int workgroups, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_ROOFLINE_H */
