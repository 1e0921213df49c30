/*
 * flashdec_kernels.h - per-step entry points and kernel timing of the
 * gfx950 FlashDecoder decode path, for unit tests and measurement.
 *
 * [FD] = "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
 * Transformers", academ.us/article/2607.14898.
 *
 * Every pointer named *_dev or passed as an operand is device memory owned by
 * the caller; `stream` is a hipStream_t (NULL = default stream).  Calls
 * enqueue work and return; errors in arguments give FD_ERR_INVALID_ARG or
 * FD_ERR_UNSUPPORTED and enqueue nothing.  bf16 values are passed as their
 * uint16 bit patterns.
 */
#ifndef FLASHDEC_KERNELS_H
#define FLASHDEC_KERNELS_H

#include "flashdec.h"

#ifdef __cplusplus
extern "C" {
#endif

/* fd_debug_read_ring - copy one ring slot exactly as it sits in device
 * memory, padding rows included (synchronises the handle's stream).
 * Passage: [FD] §3.3 Eq. 2 (one slot = one frame of L_frm keys or values);
 * the library pads a slot to n_pad = round_up(L_frm, 64) rows, which are
 * zeroed at create and never written.  Layout: keys [B G][n_pad][head_dim];
 * values transposed, [B G][head_dim][n_pad], token t in column
 * (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1) (bits 2 and 3 swapped);
 * n_pad of r_t N rows for a refinement block.  count must equal
 * B*G*n_pad*head_dim.  Codes as fd_debug_read_kv. */
fd_status fd_debug_read_ring(const fd_handle *h, int layer, int slot, int kv,
                             uint16_t *host_bf16, size_t count);

/* fd_debug_poison_ring - enqueue a fill of the token rows (not the padding)
 * of every ring slot of every block with bf16 NaN (0x7FC0), leaving the
 * bookkeeping alone, so that any read of a slot no frame has written since
 * shows up as NaN pixels.  Passage: [FD] §3.3 "Frame-by-Frame Processing"
 * (frame t attends to frames max(0, t - W_frm + 1) .. t only).
 * Returns FD_OK, FD_ERR_INVALID_ARG for NULL, FD_ERR_STATE on a broken
 * handle, FD_ERR_DEVICE when a launch fails. */
fd_status fd_debug_poison_ring(fd_handle *h);

/* fd_debug_fail_after - host-side fault injection for tests of the error
 * contract: after `launches` more kernel launches of this handle are made,
 * the next one is not made and is reported exactly as a failed launch
 * (FD_ERR_DEVICE from the call that attempted it; the handle is broken from
 * then on).  Nothing faulty ever reaches the GPU.  launches < 0 disarms.
 * Returns FD_OK, or FD_ERR_INVALID_ARG for NULL. */
fd_status fd_debug_fail_after(fd_handle *h, int64_t launches);

/* Kernel classes timed by fd_profile_read (indices of its arrays). */
enum {
  FD_K_STATE = 0,     /* ring bookkeeping (frame begin / reset) */
  FD_K_PATCHIFY = 1,  /* latent -> bf16 tokens ([FD] §3.2 Eq. 1, §4.3) */
  FD_K_INPROJ = 2,    /* tokens W_in^T + b_in ([FD] Eq. 1) */
  FD_K_LN = 3,        /* LayerNorm (pre-norm, [FD] §3.2) */
  FD_K_QKV = 4,       /* QKV GEMM + ring write ([FD] §3.3 step (2), Eq. 2) */
  FD_K_ATTN = 5,      /* attention over the ring ([FD] §3.3 step (3)) */
  FD_K_OPROJ = 6,     /* output projection + residual */
  FD_K_FC1 = 7,       /* MLP up-projection + GELU */
  FD_K_FC2 = 8,       /* MLP down-projection + residual */
  FD_K_UNPATCH = 9,   /* final projection + pixel shuffle ([FD] §3.4 Step 3) */
  FD_K_TEMPORAL = 10, /* tail: D -> r_t D linear into sub-frame tokens ([FD] Eq. 3) */
  FD_K_SPATIAL = 11,  /* tail: spatial MLP hidden layer + GELU ([FD] §3.4 Step 3) */
  FD_K_COUNT = 12
};

/* Record a HIP event pair on the handle's stream around every kernel launch
 * of fd_decode_frame / fd_reset that passes the filter, while enabled (adds
 * no synchronisation; each pair does add some time to the step). */
fd_status fd_profile_enable(fd_handle *h, int enable);

/* Restrict the launches timed while profiling: only classes k with bit k of
 * kind_mask set and, when layer >= 0, only launches of that block (launches
 * outside the blocks count as layer -1 and are then skipped; refinement block
 * r of the tail counts as layer n_layers + r).  The default is
 * kind_mask = all ones, layer = -1 (everything).  FD_ERR_INVALID_ARG for a
 * NULL handle or layer < -1; a layer >= n_layers + n_refine simply matches
 * nothing. */
fd_status fd_profile_filter(fd_handle *h, uint32_t kind_mask, int layer);

/* Synchronise the handle's stream, then write into ms[k] the summed kernel
 * time (milliseconds) and into launches[k] the launch count of every class k
 * recorded since the last read, and forget the records.  n_kinds must be
 * >= FD_K_COUNT. */
fd_status fd_profile_read(fd_handle *h, double *ms, int64_t *launches, int n_kinds);

/* out = A B^T + bias, then by epi: 0 -> fp32 store; 1 -> fp32 out += ;
 * 2 -> bf16 GELU (exact erf) store.  A: bf16 [m_rows_alloc][k] (rows >= m are
 * read, not stored); B: bf16 [n][k]; bias fp32 [n]; out [m][n] (fp32, or
 * bf16 for epi 2).  k, n, m_rows_alloc multiples of 64; m <= m_rows_alloc. */
fd_status fdk_gemm(int epi, const uint16_t *a, const uint16_t *b, const float *bias,
                   void *out, int m, int m_rows_alloc, int n, int k, void *stream);

/* Pre-sublayer norm per row of x fp32 [m][d] ([FD] §3.2), fp32 statistics,
 * bf16 out [m][d]: rms = 0, LayerNorm bf16((x - mean) / sqrt(biased var +
 * eps) * g + b); rms = 1, RMSNorm bf16(x / sqrt(mean(x^2) + eps) * g) (b
 * unused, may be NULL).  d in {64,128,192,256,384,512,768,1024,1536,2048}. */
fd_status fdk_layernorm(const float *x, int m, int d, const float *g,
                        const float *b, float eps, int rms, uint16_t *out,
                        void *stream);

/* Attention of one frame over n_frames cached frames ([FD] §3.3 step (3)):
 * out[i][j*hd + e] = sum_k softmax_k(s_ik) v_k[e] over the n_frames*n keys
 * of head j, with s_ik = q_i . k_k * ln(2) in natural units, i.e. q holds
 * queries already multiplied by log2(e)/sqrt(hd) (the library's folding).
 * Grouped-query attention ([FD] §3.2): query head j reads KV head
 * floor(j kv_heads / heads); kv_heads must divide heads.
 * q: bf16 [heads][n][hd]; k, v: bf16 [n_frames][kv_heads][n][hd], oldest
 * frame first; out: bf16 [n][heads*hd].  Frame f is placed in ring slot
 * (first_slot + f) % n_frames, exercising the ring's slot order.  splits:
 * number of key splits (1..4, head_dim 64 only), or 0 for the decoder's own
 * choice.  This entry point allocates and frees its own ring, and
 * synchronises `stream`. */
fd_status fdk_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int n_frames, int first_slot, int heads, int kv_heads,
                        int n, int hd, int splits, uint16_t *out, void *stream);

/* Bytes of device scratch fdk_attention_noalloc may use (48 MiB).  The
 * library holds one such array per GPU it runs on, until the process ends. */
#define FDK_NOALLOC_SCRATCH_BYTES (48ull << 20)

/* fdk_attention_noalloc - fdk_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, layouts and result as fdk_attention;
 * the ring, the padded queries, the ring state and the key-split partials
 * live in the library's per-GPU scratch array instead of allocations, and
 * nothing is allocated or freed (no hipMalloc, no torch allocation).
 * Needs ring 2 n_frames kv_heads round_up(n, 64) hd 2 + queries heads
 * round_up(n, 512) hd 2 + (splits > 1) splits n heads (2 hd + 16) bytes (each
 * part rounded up to 256, plus 256) within FDK_NOALLOC_SCRATCH_BYTES, else
 * FD_ERR_UNSUPPORTED and nothing is enqueued.  Asynchronous: the work is
 * enqueued on `stream` and the call returns (no synchronisation, and the
 * scratch is cleared by a fill kernel, not a memset).  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race, so the caller
 * serialises them.  Other codes as fdk_attention. */
fd_status fdk_attention_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                int n_frames, int first_slot, int heads, int kv_heads,
                                int n, int hd, int splits, uint16_t *out, void *stream);

/* fdk_mfma_probe - measurement probe of the sustained bf16 matrix-core rate
 * (not part of the decode).  Launches FDK_PROBE_WORKGROUPS workgroups of 8
 * waves (one per CU, two waves per SIMD); each wave runs `iters` rounds of
 * eight independent v_mfma_f32_32x32x16_bf16 chains on register operands,
 * all zero (zero_operands != 0) or pseudo-random in [-1, 1), with no memory
 * traffic: 2 * 32*32*16 * 8 * iters FLOPs per wave.
 * sink_dev: device fp32 [FDK_PROBE_WORKGROUPS * 512], overwritten with the
 *   accumulator sums (keeps the work alive).
 * clocks_dev: device uint64 [FDK_PROBE_WORKGROUPS * 8][2], overwritten with
 *   each wave's shader-clock (s_memtime) and 100 MHz real-time
 *   (s_memrealtime) counter deltas around its loop; their ratio times 100 MHz
 *   is the shader clock the wave ran at.
 * Asynchronous on `stream`.  FD_ERR_INVALID_ARG for NULL buffers or
 * iters <= 0, FD_ERR_DEVICE when the launch fails. */
#define FDK_PROBE_WORKGROUPS 256
fd_status fdk_mfma_probe(int zero_operands, int iters, float *sink_dev,
                         uint64_t *clocks_dev, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHDEC_KERNELS_H */
