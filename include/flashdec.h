/*
 * flashdec.h - C ABI of the MI355X (gfx950) FlashDecoder per-frame decoder.
 *
 * Source of the operation (cited by page title and section):
 *   [FD] "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
 *        Transformers", academ.us/article/2607.14898.
 *
 * The decoder turns one latent frame at a time into pixel frames, keeping a
 * fixed-size rolling key/value cache per Transformer block ([FD] §1 last
 * paragraph; §3.3 "Frame-by-Frame Processing", Eq. 2).  One call of
 * fd_decode_frame() is one step of that loop:
 *   tokens  = PixelUnshuffle(z_t) in raster order          ([FD] §3.2 Eq. 1, §4.3)
 *   H       = tokens W_in^T + b_in                          ([FD] Eq. 1)
 *   per block (pre-norm, [FD] §3.2 "Base Architecture"):
 *     [Q|K|V] = LN1(H) W_qkv^T + b_qkv; K, V of this frame replace the cache
 *     slot of frame t - W ([FD] Eq. 2); O = softmax(Q K^T / sqrt(hd)) V over
 *     every cached key, no mask ([FD] §3.3 "Attention Pattern");
 *     H += O W_o^T + b_o;  H += GELU(LN2(H) W_1^T + b_1) W_2^T + b_2
 *   pixels  = PixelShuffle(LNf(H) W_out^T + b_out)          ([FD] §3.4 Step 3)
 * The window W counts the current frame: frame t attends to frames
 * max(0, t-W+1) .. t, so frame 0 attends to itself only.
 * With n_refine > 0 the last line is replaced by the temporal-first
 * upsampling tail ([FD] §3.4), r_t = out_t, r_s = out_patch:
 *   P   = LNf(H) W_tu^T + b_tu                 [N][r_t D]    (Step 1, Eq. 3)
 *   S   = r_t N sub-frame tokens; token k N + n = columns k D .. (k+1) D - 1
 *         of P's row n (sub-frame k of this latent frame)
 *   n_refine blocks on S, each with its own ring of W latent frames of r_t N
 *         tokens (r_t W sub-frames, Step 2), same block kind as the backbone;
 *         rotary temporal positions count sub-frames (r_t t + k)
 *   pixels = PixelShuffle(GELU(LNr(S) W_s1^T + b_s1) W_s2^T + b_s2)  (Step 3)
 *         sub-frame token k N + (i W'/p + j), channel (dy r_s + dx) C + c goes
 *         to pixels[k][i r_s + dy][j r_s + dx][c].
 *
 * Conventions of this library (the pages leave them open):
 *   - LayerNorm with gain and shift, biased variance, eps = cfg.ln_eps
 *     (RMSNorm with gain only when cfg.norm = FD_NORM_RMS).
 *   - GELU(x) = x Phi(x) with erf (evaluated to within 1.5e-7 by Abramowitz
 *     and Stegun 7.1.26).  Multi-head attention, one KV head per query head,
 *     unless cfg.n_kv_heads sets grouped-query attention.
 *   - Head j owns columns j*head_dim .. (j+1)*head_dim-1 of Q and O; KV head
 *     g owns those columns of K and V.
 *   - Token n = i * (latent_w/patch) + j; token feature c*patch^2 + dy*patch
 *     + dx holds z[c][i*patch+dy][j*patch+dx].
 *   - Output channel ((tau*P + dy)*P + dx)*out_c + c of token (i, j) goes to
 *     pixels[tau][i*P+dy][j*P+dx][c], P = out_patch.
 *   - Arithmetic: bf16 operands on the matrix cores with fp32 accumulation;
 *     fp32 residual stream, LayerNorm statistics, softmax state and pixels.
 *
 * Threading: a handle is not thread-safe.  Work is enqueued on the stream
 * given at creation and runs asynchronously; results are valid after that
 * stream is synchronised.
 */
#ifndef FLASHDEC_H
#define FLASHDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
  FD_OK = 0,
  FD_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size: handle still usable */
  FD_ERR_UNSUPPORTED = -2,  /* valid config outside what the kernels support */
  FD_ERR_OOM = -3,          /* device allocation failed at create */
  FD_ERR_DEVICE = -4,       /* a HIP call failed: the handle is now broken */
  FD_ERR_STATE = -5         /* handle broken by an earlier device error */
} fd_status;

/* Largest window W the library supports. */
#define FD_MAX_WINDOW 8

/* Pre-sublayer norm types (fd_config.norm). */
#define FD_NORM_LAYER 0   /* LayerNorm: (x - mean) / sqrt(var + eps) * g + b */
#define FD_NORM_RMS 1     /* RMSNorm: x / sqrt(mean(x^2) + eps) * g ([FD] §3.2) */

/* Decoder shape.  All fields are plain int32 except ln_eps and rope_theta.
 * The last five fields select the paper's block ([FD] §3.2 "Base
 * Architecture"); all zero gives the simplified block (LayerNorm, one KV head
 * per query head, no KV-norm, no positions). */
typedef struct fd_config {
  int32_t latent_c, latent_h, latent_w;  /* C', H', W' of one latent frame */
  int32_t patch;                         /* p: PixelUnshuffle factor, 1 or 2 */
  int32_t d_model, n_heads, head_dim, mlp_dim, n_layers;
  int32_t window;                        /* W_frm: frames held in the cache */
  int32_t out_t, out_patch, out_c;       /* pixels per token: out_t x P x P x out_c */
  float ln_eps;                          /* eps of every norm */
  int32_t n_kv_heads;  /* G: K/V heads of grouped-query attention ([FD] §3.2,
                          Eq. 2); query head j reads KV head floor(j G / n_heads);
                          0 means n_heads (plain multi-head attention) */
  int32_t norm;        /* FD_NORM_LAYER or FD_NORM_RMS, for every pre-sublayer
                          norm and the final norm */
  int32_t kv_norm;     /* 1: RMS-normalise every K and V head vector (gains
                          kn_g, vn_g) before it enters the cache ([FD] §3.2) */
  int32_t rope;        /* 1: 3D rotary positions on Q and K ([FD] §3.2, §3.3
                          step (2)): head dims split (hd - 4 floor(hd/6),
                          2 floor(hd/6), 2 floor(hd/6)) between time, token row
                          and token column, consecutive pairs rotated by
                          pos * rope_theta^(-2k/d_part); temporal positions
                          relative to the window (only their differences enter
                          the scores, so keys are rotated once, when cached) */
  float rope_theta;    /* rotary base, e.g. 10000 (used when rope = 1) */
  int32_t n_refine;    /* temporal-refinement blocks of the upsampling tail
                          ([FD] §3.4); 0 = a single linear unpatchify.  With
                          n_refine > 0, out_t is r_t (<= FD_MAX_SUBFRAMES) */
  int32_t up_hidden;   /* hidden width of the tail's spatial MLP; 0 = d_model */
  int32_t batch;       /* B independent video streams decoded together, in
                          lockstep (same frame index t); each has its own
                          rings and sees only its own frames.  0 means 1 */
} fd_config;

/* Largest temporal upsampling factor r_t of the tail. */
#define FD_MAX_SUBFRAMES 8

/* One block's parameters: host fp32 arrays, Linear weights row-major
 * [out][in].  With Q = (n_heads hd) and KV = (G hd) columns, QKV = Q + 2 KV:
 * ln*_g/b [D] (b unused and may be NULL with RMSNorm); w_qkv [QKV][D] (Q
 * heads, then K heads, then V heads); b_qkv [QKV]; w_o [D][D]; b_o [D];
 * w_1 [F][D]; b_1 [F]; w_2 [D][F]; b_2 [D]; kn_g, vn_g [hd] (KV-norm gains,
 * only read when kv_norm = 1, else may be NULL). */
typedef struct fd_layer_weights {
  const float *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o;
  const float *ln2_g, *ln2_b, *w_1, *b_1, *w_2, *b_2;
  const float *kn_g, *vn_g;
} fd_layer_weights;

/* All parameters (host fp32).  w_in [D][C' p^2]; b_in [D]; layers[n_layers];
 * lnf_g/b [D] (lnf_b unused with RMSNorm); w_out [out_t P P out_c][D];
 * b_out [out_t P P out_c] (both unused, and may be NULL, when n_refine > 0).
 * The tail (read only when n_refine > 0; Hs = up_hidden or D): refine
 * [n_refine] blocks laid out as layers; w_tu [out_t D][D], b_tu [out_t D];
 * lnr_g/b [D] (lnr_b unused with RMSNorm); w_s1 [Hs][D], b_s1 [Hs];
 * w_s2 [P P out_c][Hs], b_s2 [P P out_c]. */
typedef struct fd_weights {
  const float *w_in, *b_in;
  const fd_layer_weights *layers;
  const float *lnf_g, *lnf_b, *w_out, *b_out;
  const fd_layer_weights *refine;
  const float *w_tu, *b_tu, *lnr_g, *lnr_b, *w_s1, *b_s1, *w_s2, *b_s2;
} fd_weights;

typedef struct fd_handle fd_handle;

/* Bookkeeping and memory figures of a handle (fd_query). */
typedef struct fd_info {
  int64_t frames_decoded;              /* t of the next frame */
  int32_t n_valid;                     /* frames in each block's cache */
  int32_t window;
  int32_t slot_frame[FD_MAX_WINDOW];   /* frame held by ring slot s, -1 if none */
  int32_t n_tokens, n_tokens_pad;      /* N and the padded row count of a slot */
  uint64_t arena_bytes;                /* the single device allocation */
  uint64_t weight_bytes, ring_bytes, workspace_bytes;
} fd_info;

/* fd_config_check - validate a decoder shape without touching the GPU.
 * Passage: the shape of the decoder of [FD] §3.2 "Base Architecture" and
 * §3.3 Eq. 2 (window W_frm; G KV groups; the cache holds W_frm L_frm tokens
 * per block); the upsampling tail of [FD] §3.4.
 * cfg: host memory, read during the call only.
 * Returns FD_OK; FD_ERR_INVALID_ARG for NULL or a malformed shape
 * (non-positive sizes, d_model != n_heads*head_dim, latent sides not
 * divisible by patch, window outside 1..FD_MAX_WINDOW, n_kv_heads not
 * dividing n_heads, norm not FD_NORM_LAYER / FD_NORM_RMS, negative n_refine
 * or up_hidden, out_t > FD_MAX_SUBFRAMES with n_refine > 0, batch outside
 * 0..64); FD_ERR_UNSUPPORTED for a shape the kernels do not cover (head_dim
 * not in {16, 32, 64}, d_model or mlp_dim not a multiple of 64, the QKV
 * columns (n_heads + 2G) head_dim not a multiple of 64, out_t*P*P*out_c not a
 * multiple of 64, P*out_c not a multiple of 4, patch > 2; with kv_norm or
 * rope: head_dim other than 64 or (n_heads + 2G) odd; with n_refine > 0:
 * P P out_c or up_hidden not a multiple of 64). */
fd_status fd_config_check(const fd_config *cfg);

/* fd_create - build a decoder on the current HIP device.
 * Passage: [FD] §3.3 "Frame-by-Frame Processing" (a fixed-size rolling cache
 * per block, Eq. 2) and §4.3 "Long Video Decoding" (memory constant in video
 * length): one device arena (bf16 weights, every block's K/V ring,
 * workspace) is allocated here and never grows.
 * cfg, w: host memory, read during the call only (weights are converted to
 *   bf16 and packed; the caller may free them on return).
 * stream: a hipStream_t (NULL = the default stream) on which all work of the
 *   handle is enqueued.
 * out: receives the handle, owned by the caller until fd_destroy; unchanged
 *   on error.
 * Returns FD_OK; the fd_config_check codes; FD_ERR_INVALID_ARG for a NULL
 * argument or a missing weight array; FD_ERR_OOM when the arena does not fit
 * in free device memory (nothing is left allocated); FD_ERR_DEVICE when a
 * HIP call fails (nothing is left allocated). */
fd_status fd_create(const fd_config *cfg, const fd_weights *w, void *stream,
                    fd_handle **out);

/* fd_decode_frame - one step of the streaming decoder: decode the next
 * latent frame (of every stream when batch B > 1).
 * Passage: [FD] §3.3 "Frame-by-Frame Processing" steps (1)-(3) (project the
 * frame, append its K/V and evict the oldest frame beyond W_frm, attend over
 * the whole cache) and "Attention Pattern" (no mask); §3.4 for the output
 * (linear unpatchify, or the upsampling tail with n_refine > 0).
 * latent_dev: device fp32 [B][C'][H'][W'], read-only, 4-byte aligned.
 * pixels_dev: device fp32 [B][out_t][H' P/p][W' P/p][out_c], 16-byte
 *   aligned, fully overwritten.
 * Both are owned by the caller, sized by the caller (the library cannot
 * check their extent), and must stay valid until the stream has run the
 * enqueued work.  Asynchronous: returns after enqueueing.
 * Returns FD_OK; FD_ERR_INVALID_ARG for a NULL or misaligned pointer (the
 * handle stays usable); FD_ERR_STATE on a broken handle; FD_ERR_DEVICE when
 * a launch fails (the handle is broken from then on). */
fd_status fd_decode_frame(fd_handle *h, const float *latent_dev,
                          float *pixels_dev);

/* fd_reset - forget every cached frame (of every stream): the next frame is
 * decoded as frame 0, which attends to itself only.
 * Passage: [FD] §3.3 "Frame-by-Frame Processing" (the cache of a new video
 * starts empty; W_frm counts the current frame).  Enqueued on the handle's
 * stream; the ring contents are left in place and never read again, since
 * the bookkeeping marks every slot empty.
 * Returns FD_OK; FD_ERR_INVALID_ARG for NULL; FD_ERR_STATE on a broken
 * handle; FD_ERR_DEVICE when the launch fails. */
fd_status fd_reset(fd_handle *h);

/* fd_graph_enable - record the launches of one decode step as a HIP graph
 * and replay it in every later fd_decode_frame (enable = 1), or go back to
 * plain launches (enable = 0).
 * Passage: [FD] §4.6 "Inference Optimization" item (2) (the per-frame forward
 * replayed as one captured graph).  The launch sequence is the same for every
 * frame: the ring bookkeeping lives in device memory, and the caller's
 * latent and pixel buffers are recorded there by a small launch ahead of each
 * replay, next to the frame's rotary table (paper's block).  Results are
 * bit-identical to plain launches.  Needs a handle created on a stream other
 * than the legacy default stream.  While enabled, fd_profile_enable(h, 1) is
 * refused (a replay makes no per-launch records).  Recording enqueues
 * nothing; the graph is released by fd_graph_enable(h, 0), by enabling again
 * (both first synchronise the handle's stream) and by fd_destroy.
 * Returns FD_OK; FD_ERR_INVALID_ARG for NULL or while profiling is enabled;
 * FD_ERR_UNSUPPORTED on the default stream or when the runtime cannot record
 * or instantiate the graph (the handle keeps plain launches); FD_ERR_STATE on
 * a broken handle; FD_ERR_DEVICE when that synchronisation fails (the handle
 * breaks). */
fd_status fd_graph_enable(fd_handle *h, int enable);

/* fd_destroy - synchronise the handle's stream, release the arena and the
 * handle.  Legal on a broken handle; NULL is ignored. */
void fd_destroy(fd_handle *h);

/* fd_status_string - static text for a status code ("unknown status" for a
 * value outside fd_status). */
const char *fd_status_string(fd_status s);

/* fd_query - bookkeeping of the rolling cache and the memory figures.
 * Passage: [FD] §3.3 Eq. 2 (cache of W_frm frames; frame t replaces frame
 * t - W_frm) and §4.3 "Long Video Decoding" (constant memory).
 * Synchronises the handle's stream.  info: host memory, fully written.
 * Returns FD_OK; FD_ERR_INVALID_ARG for NULL; FD_ERR_STATE on a broken
 * handle; FD_ERR_DEVICE when the read-back fails (the handle breaks). */
fd_status fd_query(const fd_handle *h, fd_info *info);

/* fd_debug_read_kv - copy the bf16 bits of one cached tensor to host memory
 * (synchronises the handle's stream).
 * Passage: [FD] §3.3 Eq. 2, the cache K_t, V_t of shape B x G x (W_frm L_frm)
 * x D_h; one slot holds one frame's L_frm rows.
 * layer < n_layers + n_refine (layers n_layers.. are the refinement blocks),
 * slot < window, kv = 0 for keys, 1 for values.  Output layout
 * [B][G][n][head_dim] whatever the internal layout (B streams, G KV heads;
 * keys as cached, i.e. after KV-norm and rotation), n = n_tokens for a
 * backbone block and out_t * n_tokens for a refinement block; count must
 * equal B*G*n*head_dim; host_bf16 is owned by the caller.
 * Returns FD_OK; FD_ERR_INVALID_ARG for NULL, an index out of range or a
 * wrong count; FD_ERR_STATE on a broken handle; FD_ERR_DEVICE when the copy
 * fails (the handle breaks). */
fd_status fd_debug_read_kv(const fd_handle *h, int layer, int slot, int kv,
                           uint16_t *host_bf16, size_t count);

#ifdef __cplusplus
}
#endif

#endif /* FLASHDEC_H */
