/*
 * gqa_decode_static.h -- the decode step without a caller-provided workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The call
 * allocates nothing; the scratch memory its kernels need (the split partials
 * and balanced tile offsets gqa_decode_step keeps in its workspace) is one
 * file-scope device array of GQA_STATIC_SCRATCH_BYTES inside the library,
 * held by every GPU the library runs on until the process ends.
 */
#ifndef GQA_DECODE_STATIC_H
#define GQA_DECODE_STATIC_H

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the library's static scratch array per GPU (32 MiB). */
#define GQA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* gqa_decode_step with the library's static scratch array as its workspace.
 * Arguments, contracts, results and errors as in gqa_decode_step (the caller
 * still passes every input and output); a descriptor whose workspace
 * (gqa_decode_workspace_size) exceeds GQA_STATIC_SCRATCH_BYTES is refused with
 * GQA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call on one
 * GPU shares that GPU's array and it keeps the last call's contents (the
 * kernels need it cleared by no one): calls that overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race. */
gqa_status_t gqa_decode_step_static(const gqa_decode_desc_t* desc, const void* q, void* k_cache,
                                    void* v_cache, const void* k_new, const void* v_new,
                                    const int32_t* lengths, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_STATIC_H */
