/*
 * csa.h -- C ABI of libcsa: the CSA/HCA Compressor (THD-packed gated-softmax
 * pooling), forward and backward, on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages):
 *   [PR5984] NVIDIA/Megatron-LM pull request 5984 page: the squashed commit
 *            log of cudnn-frontend PR #427 that brings the fused Compressor
 *            kernels over from Megatron-LM.
 *   [PR710]  cudnn-frontend pull request 710 page: ratio = 2 envelope.
 *
 * The operation ([PR5984: fused forward+backward commit; coff in {1,2}
 * commit; zero-init folding commit]).  A THD pack holds S segments of
 * token rows, segment s being rows [cu_seqlens[s], cu_seqlens[s+1]) of
 * kv and score (bf16, [total_tokens, coff*head_dim], row-major).  Each
 * segment is cut into floor(L_s / ratio) blocks of `ratio` consecutive
 * tokens; every block produces one output row, segments in order and blocks
 * in order inside a segment, so out has total_comp = sum_s floor(L_s/ratio)
 * rows.  For output column j the block's window is
 *   coff == 2: the previous block's tokens at column j (first-half columns)
 *              followed by the block's own tokens at column head_dim + j
 *              (second-half columns); a segment's first block has no
 *              previous block and uses only its own half;
 *   coff == 1: the block's own tokens at column j.
 * Each entry's logit is score + ape[position in block, column]; the window
 * is soft-maxed in fp32 per column and kv is summed under those weights;
 * the sum is rounded to bf16.  The backward produces dkv = p * dout and
 * dscore = p * dout * (kv - out_fp32) for every window entry, writes +0.0
 * into every kv/score slot no window reads, and sums dscore by (position,
 * column) into dape (fp32).
 *
 * fp32 evaluation order (fixed so results are reproducible bit for bit):
 *   x = f32(score) + ape;  m = max x;  e = EXP(x - m);  Z = e0 + e1 + ...
 *   (window order);  R = 1/Z (correctly rounded);  acc = fma chain of e*v
 *   from 0;  o = acc*R;  out = bf16_rne(o);  backward: G = R*f32(dout),
 *   a = e*G, dkv = bf16_rne(a), ds = a*(v - o), dscore = bf16_rne(ds).
 *   At ratio 2 and 4 the kernels evaluate exactly this order.  At ratio 128
 *   (windows of 128 or 256 entries) the backward sums Z and acc in chains of
 *   8 * coff consecutive entries and adds the chain sums in window order; the
 *   forward evaluates each half window (coff 2: the previous block's rows,
 *   then the own rows; coff 1: 64 rows each) with its own maximum m_h, sums
 *   16-entry chains of EXP(x - m_h) the same way and merges the halves as
 *   Z = Z_0 EXP(m_0 - M) + Z_1 EXP(m_1 - M), acc likewise, M the larger
 *   maximum ([PR5984: ratio=128 commit]: per-chunk partials with their own
 *   maxima, merged in one fixed order).  Both orders are fixed (bit-identical
 *   run to run) but differ from the single chain above by rounding: out, dkv
 *   within one bf16 ulp of the single-chain result or the error bound of the
 *   reordering and rescaling, dscore likewise, dape within 1e-5 of its
 *   largest magnitude.
 *   EXP(y) = ldexp(P7(r), k) with y clamped to >= -104, k = rint(y*log2 e),
 *   r = y - k*ln2 in two fma steps, P7 the degree-7 Taylor polynomial of
 *   e^r (coefficients fp32(1/n!)), within 1 fp32 ulp of e^y over [-104, 0];
 *   IEEE subnormals are kept.
 *
 * Conventions for every entry point:
 *   - All device pointers are caller-owned; libcsa never allocates, frees or
 *     synchronizes, and never reads device memory on the host.  Inputs are
 *     not modified and must not alias outputs.
 *   - bf16 tensors are passed as `void*` to their 16-bit elements.  Every
 *     device pointer must be 16-byte aligned (CSA_STATUS_INVALID_VALUE
 *     otherwise).  Tensors are dense, row-major.
 *   - cu_seqlens is int32 on the DEVICE, [num_segments + 1], and must satisfy
 *     cu[0] == 0, cu non-decreasing, cu[S] <= total_tokens and
 *     sum floor(L_s/ratio) == total_comp.  Empty segments are allowed.  This
 *     cannot be checked on the host without a sync: the kernels check it
 *     on the device and, if it does not hold, touch nothing but the
 *     workspace (outputs are left as they were).
 *   - total_comp is supplied by the caller (see csa_compressor_total_comp).
 *   - cu_seqlens_host (optional, may be NULL): a HOST copy of the same
 *     cu_seqlens.  When given it is validated on the host (cu[0] == 0,
 *     non-decreasing, cu[S] <= total_tokens, sum floor(L_s/ratio) ==
 *     total_comp; INVALID_VALUE otherwise) and, for packs of up to 32
 *     segments, the kernels take the segment table from their arguments and
 *     do not read the device cu_seqlens at all (the two copies must agree).
 *     Pass NULL when the device copy may change without the host knowing
 *     (e.g. a captured graph replayed with new cu_seqlens).
 *   - Work is enqueued on `stream` and is asynchronous; launch failures are
 *     returned as CSA_STATUS_LAUNCH_FAILED.
 *   - Validation is host-only and happens before any HIP call, so every
 *     rejection path works without a GPU.
 *   - Thread-safe: no global mutable state besides the thread-local error
 *     text and tuning knobs read once from the environment.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
    CSA_STATUS_SUCCESS = 0,
    /* a null or misaligned pointer, a negative size, inconsistent sizes
     * (e.g. total_comp * ratio > total_tokens), an undersized output */
    CSA_STATUS_INVALID_VALUE = 1,
    /* outside the validated envelope: ratio not in {2, 4, 128}, coff not in
     * {1, 2}, head_dim not in [1, 1024] (a multiple of 64 at ratio 128),
     * or one of
     * (total_tokens+1)*coff*head_dim, total_comp*head_dim,
     * ratio*coff*head_dim not below 2^31 (each checked on its own) */
    CSA_STATUS_NOT_SUPPORTED = 2,
    /* workspace_bytes below the size the *_workspace_size query returns */
    CSA_STATUS_WORKSPACE_TOO_SMALL = 3,
    /* a kernel launch failed (hipGetLastError after the launch) */
    CSA_STATUS_LAUNCH_FAILED = 4,
    /* reserved: the current device could not be queried */
    CSA_STATUS_DEVICE_ERROR = 5
} csa_status_t;

/* Static text for a status code; never NULL. */
const char* csa_status_string(csa_status_t status);

/* Human-readable detail of the last failing call made on this thread
 * (empty string if none).  The pointer stays valid until the next libcsa
 * call on the same thread. */
const char* csa_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t csa_version(void);

/* Host helper: total_comp = sum_s floor((cu[s+1]-cu[s]) / ratio) from a HOST
 * copy of cu_seqlens [num_segments + 1].  INVALID_VALUE if a pointer is null,
 * ratio < 1, num_segments < 0, cu[0] != 0 or cu decreases.  ([PR5984:
 * zero-init folding commit] names this count total_comp.) */
csa_status_t csa_compressor_total_comp(const int32_t* cu_seqlens_host, int32_t num_segments,
                                       int32_t ratio, int64_t* total_comp);

/* Envelope check without any buffer ([PR5984: review-feedback commit and
 * coff commit], [PR710: What]): SUCCESS, NOT_SUPPORTED (envelope, see the
 * status codes) or INVALID_VALUE (negative sizes, total_comp > 0 with
 * total_tokens < ratio, total_comp * ratio > total_tokens). */
csa_status_t csa_compressor_check_support(int32_t ratio, int32_t coff, int32_t head_dim,
                                          int32_t num_segments, int64_t total_tokens,
                                          int64_t total_comp);

/* Workspace bytes the forward / backward need for this problem (0 is
 * possible; the size depends on the problem, not on the device).  The workspace is device memory, 16-byte aligned,
 * caller-owned, uninitialized on entry, and may be reused across calls that
 * are stream-ordered; two calls running concurrently need two workspaces. */
csa_status_t csa_compressor_fwd_workspace_size(int32_t ratio, int32_t coff, int32_t head_dim,
                                               int32_t num_segments, int64_t total_tokens,
                                               int64_t total_comp, size_t* bytes);
csa_status_t csa_compressor_bwd_workspace_size(int32_t ratio, int32_t coff, int32_t head_dim,
                                               int32_t num_segments, int64_t total_tokens,
                                               int64_t total_comp, size_t* bytes);

/* Forward ([PR5984: fused forward+backward commit]).
 *   kv, score  bf16 [total_tokens, coff*head_dim]   (device, read)
 *   ape        fp32 [ratio, coff*head_dim]           (device, read)
 *   cu_seqlens int32 [num_segments + 1]              (device, read)
 *   cu_seqlens_host int32 [num_segments + 1]         (host, optional)
 *   out        bf16 [total_comp, head_dim]           (device, fully written)
 * total_comp == 0 enqueues nothing. */
csa_status_t csa_compressor_fwd(const void* kv, const void* score, const float* ape,
                                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                int32_t num_segments, int64_t total_tokens, int64_t total_comp,
                                int32_t ratio, int32_t coff, int32_t head_dim,
                                void* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Backward ([PR5984: fused forward+backward commit; zero-init folding
 * commit]).  Inputs as the forward plus
 *   dout       bf16 [total_comp, head_dim]                  (device, read)
 * Outputs, all fully overwritten (no prefill needed; NaN-filled buffers are
 * fine):
 *   dkv, dscore bf16 [total_tokens, coff*head_dim]: the gradient on every
 *              slot some window reads, bit pattern 0x0000 (+0.0) on every
 *              slot none reads (the first-half columns of each segment's
 *              last block at coff == 2, the seqlen % ratio tail rows, the
 *              rows of segments shorter than ratio, the rows past
 *              cu_seqlens[S]);
 *   dape       fp32 [ratio, coff*head_dim].
 * out/dkv/dscore are deterministic (bit-identical run to run).  dape is
 * reduced in a fixed order and is bit-identical run to run for a given
 * device and problem; `deterministic` is accepted for forward compatibility
 * (0 would permit an unordered reduction) and does not change the result:
 * the library has only the fixed-order reduction.  total_comp == 0 still
 * writes all zeros to dkv/dscore/dape. */
csa_status_t csa_compressor_bwd(const void* kv, const void* score, const float* ape,
                                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                int32_t num_segments, int64_t total_tokens, int64_t total_comp,
                                int32_t ratio, int32_t coff, int32_t head_dim,
                                const void* dout, void* dkv, void* dscore, float* dape,
                                int32_t deterministic, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* The backward's two stages, for callers that schedule them separately
 * (e.g. to time the gradient kernel alone).  csa_compressor_bwd is exactly
 * bwd_grads followed by bwd_dape_reduce on the same stream and workspace.
 *   bwd_grads: writes dkv and dscore in full and per-workgroup dAPE partial
 *              sums into the workspace.
 *   bwd_dape_reduce: sums those partials in a fixed order into dape.
 * Both take the same problem description and workspace as the full call;
 * bwd_dape_reduce must run after bwd_grads of the same problem on the same
 * workspace, with nothing writing the workspace in between. */
csa_status_t csa_compressor_bwd_grads(const void* kv, const void* score, const float* ape,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                      int32_t num_segments, int64_t total_tokens, int64_t total_comp,
                                      int32_t ratio, int32_t coff, int32_t head_dim,
                                      const void* dout, void* dkv, void* dscore,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
csa_status_t csa_compressor_bwd_dape_reduce(int32_t ratio, int32_t coff, int32_t head_dim,
                                            int32_t num_segments, int64_t total_tokens,
                                            int64_t total_comp, float* dape,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* The backward (same arguments, same results, bit for bit, as
 * csa_compressor_bwd) without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It calls no allocating routine; the
 * workspace lives in scratch memory owned by the library: one array of
 * CSA_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load on that
 * GPU until the process ends, its address looked up on the first call on
 * each device (the device current at the call is used).
 *   - A problem whose workspace (csa_compressor_bwd_workspace_size) exceeds
 *     CSA_NOALLOC_SCRATCH_BYTES is rejected with
 *     CSA_STATUS_WORKSPACE_TOO_SMALL before anything is enqueued; every
 *     ratio 2 / 4 problem of the envelope fits at the default launch shapes,
 *     ratio 128 up to about 32 MiB of dAPE partials.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents; nothing in it has to start at zero.  Calls that
 *     overlap on one GPU (different streams, or different host threads,
 *     without ordering between them) race on it and give undefined results.
 *   - CSA_STATUS_DEVICE_ERROR if the scratch of the current device cannot be
 *     located. */
#define CSA_NOALLOC_SCRATCH_BYTES (40u * 1024u * 1024u)
csa_status_t csa_compressor_bwd_noalloc(const void* kv, const void* score, const float* ape,
                                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                        int32_t num_segments, int64_t total_tokens, int64_t total_comp,
                                        int32_t ratio, int32_t coff, int32_t head_dim,
                                        const void* dout, void* dkv, void* dscore, float* dape,
                                        int32_t deterministic, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
