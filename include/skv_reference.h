/*
 * skv_reference.h -- bandwidth references of libsparsekv.so, used to place
 * the decode kernels against what this GPU delivers for the same bytes.
 * They carry none of the method's arithmetic: each only reads device memory
 * and folds what it read into a value that is almost never stored, so the
 * reads cannot be optimised away.
 *
 * Conventions as in sparsekv.h: device pointers owned by the caller,
 * asynchronous on `stream`, SKV_OK / SKV_EINVAL / SKV_EFAULT / SKV_EIO.
 */
#ifndef SKV_REFERENCE_H
#define SKV_REFERENCE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * skv_ref_stream_read -- read `bytes` of device memory at `buf` once, in
 * address order, with the whole GPU: 1024 blocks of 512 threads, 16-byte
 * loads in a grid-stride loop.  The plain streaming read of a launch of this
 * size.
 *   buf    16-byte aligned; bytes a positive multiple of 16.
 *   sink   uint32 [1024]; a word may be written (only if a block's XOR of its
 *          data equals 0x5ca1ab1e), so its contents afterwards are unspecified.
 */
int skv_ref_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                        hipStream_t stream);

/*
 * skv_ref_gather_read -- read the K and V rows of n page-heads of a paged
 * cache, as an attention decode over them must: item i = (block
 * items[3i], kv head items[3i+1], valid rows items[3i+2]), whose rows
 * t < valid rows are read for K and for V (D bf16 each, 16-byte loads, one
 * wave per item, up to 4096 blocks of 4 waves, so that many short waves keep
 * the most reads in flight; a row past the valid count reads row 0 of the
 * same page so the loads stay unconditional).  The gather-only rate for a
 * decode's own list of page-heads.
 *   kv_cache bf16 [2, num_blocks, page_size, H_kv, D]; page_size 16,
 *            D in {64, 128}.
 *   items    int32 [n, 3]; block < num_blocks, kv head < H_kv, rows <= 16
 *            (trusted, as block ids are elsewhere).
 *   sink     uint32 [256]; as skv_ref_stream_read.
 */
int skv_ref_gather_read(const uint16_t *kv_cache, int64_t num_blocks,
                        int page_size, int H_kv, int D, const int32_t *items,
                        int64_t n, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKV_REFERENCE_H */
