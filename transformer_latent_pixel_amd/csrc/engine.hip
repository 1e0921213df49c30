// Decoder engine and the C ABI of flashdec.h / flashdec_kernels.h.
//
// [FD] = "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
// Transformers" (academ.us/article/2607.14898).
//
// One device arena is allocated at create and carved into: bf16 weights
// (row-major [out][in], the GEMM's B operand as is), fp32 biases and norm
// parameters, per-block K and V^T rings ([FD] §3.3 Eq. 2: W frames of N
// tokens; the refinement blocks of the upsampling tail, [FD] §3.4, hold W
// frames of r_t N sub-frame tokens), the activation workspace (rows padded to a multiple of 256 so that
// GEMM tiles never read past an allocation), and the ring bookkeeping.  The
// arena never grows, so device memory is constant in video length
// ([FD] §4.3 "Long Video Decoding").
#include <math.h>
#include <string.h>

#include <new>
#include <vector>

#include "fd_common.h"
#include "flashdec_kernels.h"

using namespace fd;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
uint16_t host_f2bf(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

bool ln_dim_ok(int d) {
  switch (d) {
    case 64: case 128: case 192: case 256: case 384: case 512: case 768:
    case 1024: case 1536: case 2048:
      return true;
    default:
      return false;
  }
}

struct LayerPtrs {
  float *ln1_g, *ln1_b, *b_qkv, *b_o, *ln2_g, *ln2_b, *b_1, *b_2;
  float *kn_g, *vn_g;
  uint16_t *w_qkv, *w_o, *w_1, *w_2;
  uint16_t *ring_k, *ring_vt;
};

// Bump allocator over the arena; a first pass with base = nullptr sizes it.
struct Carver {
  uint8_t* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    off = round_up(off, kAlign);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

}  // namespace

struct fd_handle {
  fd_config cfg;
  hipStream_t stream = nullptr;
  int device = 0;
  bool broken = false;

  // Derived sizes.  m_rows and q_rows cover the larger of the backbone's N
  // tokens and the tail's N4 = r_t N sub-frame tokens.
  int N = 0, n_pad = 0, m_rows = 0, q_rows = 0, k_in = 0, k_in_pad = 0;
  int R = 0, N4 = 0, n4_pad = 0, up_h = 0, sub_c = 0, splits_r = 1;
  int B = 1;                        // streams decoded together
  int D = 0, F = 0, heads = 0, hd = 0, L = 0, W = 0, c_out = 0;
  int kv_heads = 0, qkv_n = 0;      // KV heads G; QKV columns (heads + 2G) hd
  int tok_h = 0, tok_w = 0, pix_h = 0, pix_w = 0;
  bool rms = false, kv_norm = false, rope = false;
  int64_t host_t = 0;               // frame index of the next decode (rotary angles)
  float2 *rope_h = nullptr, *rope_w = nullptr;   // per-token rotary cos/sin
  float2* rope_t = nullptr;         // this frame's temporal cos/sin [kRopeRows][12]
  float q_scale = 0.0f;

  uint8_t* arena = nullptr;
  size_t arena_bytes = 0, weight_bytes = 0, ring_bytes = 0, ws_bytes = 0;

  uint16_t* w_in = nullptr;
  float* b_in = nullptr;
  std::vector<LayerPtrs> layers;
  float *lnf_g = nullptr, *lnf_b = nullptr, *b_out = nullptr;
  uint16_t* w_out = nullptr;
  // Upsampling tail: refinement blocks, temporal linear, norm, spatial MLP.
  std::vector<LayerPtrs> rlayers;
  uint16_t *w_tu = nullptr, *w_s1 = nullptr, *w_s2 = nullptr;
  float *b_tu = nullptr, *lnr_g = nullptr, *lnr_b = nullptr, *b_s1 = nullptr, *b_s2 = nullptr;

  uint16_t *x = nullptr, *a = nullptr, *q = nullptr, *o = nullptr, *u = nullptr;
  float* h = nullptr;
  DeviceState* state = nullptr;
  // Attention key splits and their partial outputs (only when splits > 1).
  int splits = 1;
  uint16_t* part_o = nullptr;
  float* part_ml = nullptr;

  // Kernel timing with HIP events on the handle's stream: only launches of
  // a class in prof_mask, and of block prof_layer when that is >= 0
  // (launches outside the blocks have layer -1).
  // Host-side fault injection (fd_debug_fail_after): launches still allowed
  // before one is reported failed instead of being made; -1 = off.
  int64_t fail_after = -1;

  bool profiling = false;
  uint32_t prof_mask = 0xFFFFFFFFu;
  int prof_layer = -1;
  int cur_layer = -1;
  struct Rec { int kind; hipEvent_t start, stop; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> event_pool;
  size_t pool_used = 0;

  // fd_graph_enable: the recorded launches of one frame (after the rotary
  // table), replayed by fd_decode_frame while set.
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;
};

namespace {

// Carve every region; with h->arena == nullptr only the sizes are computed.
void carve(fd_handle* h) {
  Carver cv{h->arena};
  const int D = h->D, F = h->F;
  h->w_in = cv.take<uint16_t>((size_t)D * h->k_in_pad);
  h->b_in = cv.take<float>(D);
  h->layers.resize(h->L);
  h->rlayers.resize(h->R);
  auto carve_block = [&](LayerPtrs& l) {
    l.ln1_g = cv.take<float>(D); l.ln1_b = cv.take<float>(D);
    l.w_qkv = cv.take<uint16_t>((size_t)h->qkv_n * D); l.b_qkv = cv.take<float>(h->qkv_n);
    l.kn_g = h->kv_norm ? cv.take<float>(h->hd) : nullptr;
    l.vn_g = h->kv_norm ? cv.take<float>(h->hd) : nullptr;
    l.w_o = cv.take<uint16_t>((size_t)D * D); l.b_o = cv.take<float>(D);
    l.ln2_g = cv.take<float>(D); l.ln2_b = cv.take<float>(D);
    l.w_1 = cv.take<uint16_t>((size_t)F * D); l.b_1 = cv.take<float>(F);
    l.w_2 = cv.take<uint16_t>((size_t)D * F); l.b_2 = cv.take<float>(D);
  };
  for (auto& l : h->layers) carve_block(l);
  h->lnf_g = cv.take<float>(D); h->lnf_b = cv.take<float>(D);
  if (h->R == 0) {
    h->w_out = cv.take<uint16_t>((size_t)h->c_out * D);
    h->b_out = cv.take<float>(h->c_out);
  } else {
    for (auto& l : h->rlayers) carve_block(l);
    const int rt = h->cfg.out_t;
    h->w_tu = cv.take<uint16_t>((size_t)rt * D * D); h->b_tu = cv.take<float>((size_t)rt * D);
    h->lnr_g = cv.take<float>(D); h->lnr_b = cv.take<float>(D);
    h->w_s1 = cv.take<uint16_t>((size_t)h->up_h * D); h->b_s1 = cv.take<float>(h->up_h);
    h->w_s2 = cv.take<uint16_t>((size_t)h->sub_c * h->up_h); h->b_s2 = cv.take<float>(h->sub_c);
  }
  if (h->rope) {
    h->rope_h = cv.take<float2>((size_t)h->tok_h * 10);
    h->rope_w = cv.take<float2>((size_t)h->tok_w * 10);
    h->rope_t = cv.take<float2>((size_t)kRopeRows * 12);
  }
  h->weight_bytes = round_up(cv.off, kAlign);

  const size_t ring_elems = (size_t)h->W * h->B * h->kv_heads * h->n_pad * h->hd;
  const size_t ring4_elems = (size_t)h->W * h->B * h->kv_heads * h->n4_pad * h->hd;
  const size_t r0 = round_up(cv.off, kAlign);
  for (auto& l : h->layers) {
    l.ring_k = cv.take<uint16_t>(ring_elems);
    l.ring_vt = cv.take<uint16_t>(ring_elems);
  }
  for (auto& l : h->rlayers) {
    l.ring_k = cv.take<uint16_t>(ring4_elems);
    l.ring_vt = cv.take<uint16_t>(ring4_elems);
  }
  h->ring_bytes = round_up(cv.off, kAlign) - r0;

  const size_t w0 = round_up(cv.off, kAlign);
  const size_t M = h->m_rows;
  h->x = cv.take<uint16_t>(M * h->k_in_pad);
  h->h = cv.take<float>(M * D);
  h->a = cv.take<uint16_t>(M * D);
  h->q = cv.take<uint16_t>((size_t)h->B * h->heads * h->q_rows * h->hd);
  h->o = cv.take<uint16_t>(M * D);
  h->u = cv.take<uint16_t>(M * (size_t)(F > h->up_h ? F : h->up_h));
  h->state = cv.take<DeviceState>(1);
  // Attention partials for the larger of the two token sets that split keys.
  // part_o [splits][rows][B heads hd], part_ml [splits][B heads][rows][4].
  const size_t pr_b = h->splits > 1 ? (size_t)h->splits * h->N : 0;
  const size_t pr_r = h->splits_r > 1 ? (size_t)h->splits_r * h->N4 : 0;
  const size_t part_rows = (pr_b > pr_r ? pr_b : pr_r) * h->B;
  if (part_rows) {
    h->part_o = cv.take<uint16_t>(part_rows * D);
    h->part_ml = cv.take<float>(part_rows * h->heads * 4);
  }
  h->ws_bytes = round_up(cv.off, kAlign) - w0;
  h->arena_bytes = round_up(cv.off, kAlign);
}

fd_status upload_bf16(const float* src, uint16_t* dst, int rows, int cols,
                      int ld_dst, std::vector<uint16_t>& tmp) {
  tmp.assign((size_t)rows * ld_dst, 0);
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      tmp[(size_t)r * ld_dst + c] = host_f2bf(src[(size_t)r * cols + c]);
  return hipMemcpy(dst, tmp.data(), tmp.size() * 2, hipMemcpyHostToDevice) == hipSuccess
             ? FD_OK : FD_ERR_DEVICE;
}

fd_status upload_f32(const float* src, float* dst, size_t n) {
  return hipMemcpy(dst, src, n * 4, hipMemcpyHostToDevice) == hipSuccess ? FD_OK
                                                                          : FD_ERR_DEVICE;
}

// Rotary frequencies of pair k in an axis part of `size` head dims:
// theta^(-2k/size) ([FD] §3.2 3D-RoPE; split 24/20/20 of head_dim 64).
double rope_freq(double theta, int k, int size) { return pow(theta, -2.0 * k / size); }

// Per-token cos/sin of the row pairs (rope_h[i][k], k < 10) and column pairs
// (rope_w[j][k]), computed in double on the host.
fd_status upload_rope_tables(fd_handle* h) {
  const double theta = h->cfg.rope_theta;
  std::vector<float2> th((size_t)h->tok_h * 10), tw((size_t)h->tok_w * 10);
  for (int i = 0; i < h->tok_h; ++i)
    for (int k = 0; k < 10; ++k) {
      const double a = i * rope_freq(theta, k, 20);
      th[(size_t)i * 10 + k] = make_float2((float)cos(a), (float)sin(a));
    }
  for (int j = 0; j < h->tok_w; ++j)
    for (int k = 0; k < 10; ++k) {
      const double a = j * rope_freq(theta, k, 20);
      tw[(size_t)j * 10 + k] = make_float2((float)cos(a), (float)sin(a));
    }
  if (hipMemcpy(h->rope_h, th.data(), th.size() * sizeof(float2), hipMemcpyHostToDevice) !=
          hipSuccess ||
      hipMemcpy(h->rope_w, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice) !=
          hipSuccess)
    return FD_ERR_DEVICE;
  return FD_OK;
}

hipEvent_t take_event(fd_handle* h) {
  if (h->pool_used == h->event_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    h->event_pool.push_back(e);
  }
  return h->event_pool[h->pool_used++];
}

// Launch wrapper: records a start/stop event pair around the launch when
// profiling is on, and turns a launch error into a broken handle.
template <typename Fn>
fd_status run(fd_handle* h, int kind, Fn&& fn) {
  if (h->fail_after == 0) {
    // Injected failure: the launch is not made, and the handle breaks exactly
    // as after a failed launch.
    h->fail_after = -1;
    h->broken = true;
    return FD_ERR_DEVICE;
  }
  if (h->fail_after > 0) --h->fail_after;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool rec = h->profiling && ((h->prof_mask >> kind) & 1u) &&
                   (h->prof_layer < 0 || h->prof_layer == h->cur_layer);
  if (rec) {
    e0 = take_event(h);
    e1 = take_event(h);
    // A pair whose start could not be recorded is dropped, not reported.
    if (e0 && hipEventRecord(e0, h->stream) != hipSuccess) e0 = nullptr;
  }
  hipError_t err = fn();
  if (rec && e0 && e1 && hipEventRecord(e1, h->stream) == hipSuccess)
    h->recs.push_back({kind, e0, e1});
  if (err != hipSuccess) {
    h->broken = true;
    return FD_ERR_DEVICE;
  }
  return FD_OK;
}

#define FD_TRY(expr)                   \
  do {                                 \
    fd_status st_ = (expr);            \
    if (st_ != FD_OK) return st_;      \
  } while (0)

EpiParams epi_plain(const float* bias, float* f32, uint16_t* bf, int ldo) {
  EpiParams e{};
  e.bias = bias;
  e.out_f32 = f32;
  e.out_bf16 = bf;
  e.ldo = ldo;
  return e;
}

}  // namespace

extern "C" {

const char* fd_status_string(fd_status s) {
  switch (s) {
    case FD_OK: return "ok";
    case FD_ERR_INVALID_ARG: return "invalid argument";
    case FD_ERR_UNSUPPORTED: return "unsupported configuration";
    case FD_ERR_OOM: return "device out of memory";
    case FD_ERR_DEVICE: return "device error";
    case FD_ERR_STATE: return "handle broken by an earlier device error";
  }
  return "unknown status";
}

fd_status fd_config_check(const fd_config* c) {
  if (!c) return FD_ERR_INVALID_ARG;
  if (c->latent_c <= 0 || c->latent_h <= 0 || c->latent_w <= 0 || c->patch <= 0 ||
      c->d_model <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->mlp_dim <= 0 ||
      c->n_layers <= 0 || c->out_t <= 0 || c->out_patch <= 0 || c->out_c <= 0)
    return FD_ERR_INVALID_ARG;
  if (c->window < 1 || c->window > FD_MAX_WINDOW) return FD_ERR_INVALID_ARG;
  if (c->d_model != c->n_heads * c->head_dim) return FD_ERR_INVALID_ARG;
  if (c->latent_h % c->patch || c->latent_w % c->patch) return FD_ERR_INVALID_ARG;
  if (!(c->ln_eps > 0.0f) || !isfinite(c->ln_eps)) return FD_ERR_INVALID_ARG;
  if (c->patch > 2) return FD_ERR_UNSUPPORTED;
  if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64) return FD_ERR_UNSUPPORTED;
  if (c->n_kv_heads < 0 || (c->n_kv_heads && c->n_heads % c->n_kv_heads))
    return FD_ERR_INVALID_ARG;
  if (c->norm != FD_NORM_LAYER && c->norm != FD_NORM_RMS) return FD_ERR_INVALID_ARG;
  if ((c->kv_norm != 0 && c->kv_norm != 1) || (c->rope != 0 && c->rope != 1))
    return FD_ERR_INVALID_ARG;
  if (c->rope && (!(c->rope_theta > 1.0f) || !isfinite(c->rope_theta)))
    return FD_ERR_INVALID_ARG;
  if (c->kv_norm || c->rope) {
    // the per-head epilogue works on 64-column heads in waves of >= 64 columns
    const int g = c->n_kv_heads ? c->n_kv_heads : c->n_heads;
    if (c->head_dim != 64 || (c->n_heads + 2 * g) % 2) return FD_ERR_UNSUPPORTED;
  }
  if (c->n_refine < 0 || c->up_hidden < 0) return FD_ERR_INVALID_ARG;
  if (c->batch < 0 || c->batch > 64) return FD_ERR_INVALID_ARG;
  if (c->n_refine > 0 && c->out_t > FD_MAX_SUBFRAMES) return FD_ERR_INVALID_ARG;
  if (c->d_model % 64 || c->mlp_dim % 64 || !ln_dim_ok(c->d_model)) return FD_ERR_UNSUPPORTED;
  {
    // the QKV GEMM's (heads + 2G) head_dim output columns come in 64-column tiles
    const long g = c->n_kv_heads ? c->n_kv_heads : c->n_heads;
    if (((long)c->n_heads + 2 * g) * c->head_dim % 64) return FD_ERR_UNSUPPORTED;
  }
  const long c_out = (long)c->out_t * c->out_patch * c->out_patch * c->out_c;
  if (c_out % 64 || c_out > (1 << 20)) return FD_ERR_UNSUPPORTED;
  if ((c->out_patch * c->out_c) % 4) return FD_ERR_UNSUPPORTED;   // float4 pixel stores
  const long ntok = (long)(c->latent_h / c->patch) * (c->latent_w / c->patch);
  if (ntok > (1 << 20)) return FD_ERR_UNSUPPORTED;
  if (c->n_refine > 0) {
    // the spatial MLP's two GEMMs need 64-multiples for N and K
    if ((c->out_patch * c->out_patch * c->out_c) % 64 || c->up_hidden % 64)
      return FD_ERR_UNSUPPORTED;
    if (ntok * c->out_t > (1 << 20)) return FD_ERR_UNSUPPORTED;
  }
  const long rows = (c->batch ? c->batch : 1) * ntok * (c->n_refine > 0 ? c->out_t : 1);
  if (rows > (1 << 21)) return FD_ERR_UNSUPPORTED;
  return FD_OK;
}

fd_status fd_create(const fd_config* cfg, const fd_weights* w, void* stream,
                    fd_handle** out) {
  if (!cfg || !w || !out) return FD_ERR_INVALID_ARG;
  FD_TRY(fd_config_check(cfg));
  const bool tail = cfg->n_refine > 0;
  if (!w->w_in || !w->b_in || !w->layers || !w->lnf_g) return FD_ERR_INVALID_ARG;
  if (!tail && (!w->w_out || !w->b_out)) return FD_ERR_INVALID_ARG;
  const bool rms = cfg->norm == FD_NORM_RMS;
  if (!rms && !w->lnf_b) return FD_ERR_INVALID_ARG;
  auto block_ok = [&](const fd_layer_weights& lw) {
    if (!lw.ln1_g || !lw.w_qkv || !lw.b_qkv || !lw.w_o || !lw.b_o ||
        !lw.ln2_g || !lw.w_1 || !lw.b_1 || !lw.w_2 || !lw.b_2)
      return false;
    if (!rms && (!lw.ln1_b || !lw.ln2_b)) return false;
    if (cfg->kv_norm && (!lw.kn_g || !lw.vn_g)) return false;
    return true;
  };
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!block_ok(w->layers[l])) return FD_ERR_INVALID_ARG;
  if (tail) {
    if (!w->refine || !w->w_tu || !w->b_tu || !w->lnr_g || (!rms && !w->lnr_b) || !w->w_s1 ||
        !w->b_s1 || !w->w_s2 || !w->b_s2)
      return FD_ERR_INVALID_ARG;
    for (int r = 0; r < cfg->n_refine; ++r)
      if (!block_ok(w->refine[r])) return FD_ERR_INVALID_ARG;
  }

  fd_handle* h = new (std::nothrow) fd_handle();
  if (!h) return FD_ERR_OOM;
  h->cfg = *cfg;
  h->stream = (hipStream_t)stream;
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return FD_ERR_DEVICE; }

  const int p = cfg->patch;
  h->tok_w = cfg->latent_w / p;
  h->tok_h = cfg->latent_h / p;
  h->N = h->tok_h * h->tok_w;
  h->n_pad = (int)round_up(h->N, 64);
  h->B = cfg->batch ? cfg->batch : 1;
  h->R = cfg->n_refine;
  h->N4 = h->R ? cfg->out_t * h->N : 0;
  h->n4_pad = (int)round_up(h->N4, 64);
  const int rows = h->N4 > h->N ? h->N4 : h->N;   // token rows of one stream
  h->m_rows = (int)round_up((size_t)h->B * rows, 256);
  h->q_rows = (int)round_up(rows, 512);      // attention reads Q in 512-row tiles
  h->up_h = cfg->up_hidden ? cfg->up_hidden : cfg->d_model;
  h->sub_c = cfg->out_patch * cfg->out_patch * cfg->out_c;
  h->k_in = cfg->latent_c * p * p;
  h->k_in_pad = (int)round_up(h->k_in, 64);
  h->D = cfg->d_model;
  h->F = cfg->mlp_dim;
  h->heads = cfg->n_heads;
  h->hd = cfg->head_dim;
  h->kv_heads = cfg->n_kv_heads ? cfg->n_kv_heads : cfg->n_heads;
  h->qkv_n = (h->heads + 2 * h->kv_heads) * h->hd;
  h->rms = cfg->norm == FD_NORM_RMS;
  h->kv_norm = cfg->kv_norm != 0;
  h->rope = cfg->rope != 0;
  h->L = cfg->n_layers;
  h->W = cfg->window;
  h->c_out = cfg->out_t * cfg->out_patch * cfg->out_patch * cfg->out_c;
  h->pix_h = (cfg->latent_h / p) * cfg->out_patch;
  h->pix_w = h->tok_w * cfg->out_patch;
  // Scores in log2 units: Q is scaled by log2(e) / sqrt(head_dim).
  h->q_scale = (float)(1.4426950408889634 / sqrt((double)h->hd));

  h->splits = attention_splits(h->B * h->heads, h->N, h->hd);
  h->splits_r = h->R ? attention_splits(h->B * h->heads, h->N4, h->hd) : 1;
  carve(h);                                   // sizes only
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) { delete h; return FD_ERR_DEVICE; }
  if (h->arena_bytes > free_b) { delete h; return FD_ERR_OOM; }
  void* mem = nullptr;
  if (hipMalloc(&mem, h->arena_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return FD_ERR_OOM;
  }
  h->arena = (uint8_t*)mem;
  carve(h);                                   // real pointers

  fd_status st = FD_OK;
  // Zero everything: K/V ring padding rows and activation padding rows must
  // read as 0 (they are never written).
  if (hipMemset(h->arena, 0, h->arena_bytes) != hipSuccess) st = FD_ERR_DEVICE;
  std::vector<uint16_t> tmp;
  const int D = h->D, F = h->F;
  if (st == FD_OK) st = upload_bf16(w->w_in, h->w_in, D, h->k_in, h->k_in_pad, tmp);
  if (st == FD_OK) st = upload_f32(w->b_in, h->b_in, D);
  auto upload_block = [&](const fd_layer_weights& lw, LayerPtrs& d) {
    fd_status st = upload_f32(lw.ln1_g, d.ln1_g, D);
    if (st == FD_OK && lw.ln1_b) st = upload_f32(lw.ln1_b, d.ln1_b, D);
    if (st == FD_OK) st = upload_bf16(lw.w_qkv, d.w_qkv, h->qkv_n, D, D, tmp);
    if (st == FD_OK) st = upload_f32(lw.b_qkv, d.b_qkv, h->qkv_n);
    if (st == FD_OK && h->kv_norm) st = upload_f32(lw.kn_g, d.kn_g, h->hd);
    if (st == FD_OK && h->kv_norm) st = upload_f32(lw.vn_g, d.vn_g, h->hd);
    if (st == FD_OK) st = upload_bf16(lw.w_o, d.w_o, D, D, D, tmp);
    if (st == FD_OK) st = upload_f32(lw.b_o, d.b_o, D);
    if (st == FD_OK) st = upload_f32(lw.ln2_g, d.ln2_g, D);
    if (st == FD_OK && lw.ln2_b) st = upload_f32(lw.ln2_b, d.ln2_b, D);
    if (st == FD_OK) st = upload_bf16(lw.w_1, d.w_1, F, D, D, tmp);
    if (st == FD_OK) st = upload_f32(lw.b_1, d.b_1, F);
    if (st == FD_OK) st = upload_bf16(lw.w_2, d.w_2, D, F, F, tmp);
    if (st == FD_OK) st = upload_f32(lw.b_2, d.b_2, D);
    return st;
  };
  for (int l = 0; l < h->L && st == FD_OK; ++l) st = upload_block(w->layers[l], h->layers[l]);
  if (st == FD_OK) st = upload_f32(w->lnf_g, h->lnf_g, D);
  if (st == FD_OK && w->lnf_b) st = upload_f32(w->lnf_b, h->lnf_b, D);
  if (st == FD_OK && h->rope) st = upload_rope_tables(h);
  if (h->R == 0) {
    if (st == FD_OK) st = upload_bf16(w->w_out, h->w_out, h->c_out, D, D, tmp);
    if (st == FD_OK) st = upload_f32(w->b_out, h->b_out, h->c_out);
  } else {
    const int rt = cfg->out_t;
    for (int r = 0; r < h->R && st == FD_OK; ++r) st = upload_block(w->refine[r], h->rlayers[r]);
    if (st == FD_OK) st = upload_bf16(w->w_tu, h->w_tu, rt * D, D, D, tmp);
    if (st == FD_OK) st = upload_f32(w->b_tu, h->b_tu, (size_t)rt * D);
    if (st == FD_OK) st = upload_f32(w->lnr_g, h->lnr_g, D);
    if (st == FD_OK && w->lnr_b) st = upload_f32(w->lnr_b, h->lnr_b, D);
    if (st == FD_OK) st = upload_bf16(w->w_s1, h->w_s1, h->up_h, D, D, tmp);
    if (st == FD_OK) st = upload_f32(w->b_s1, h->b_s1, h->up_h);
    if (st == FD_OK) st = upload_bf16(w->w_s2, h->w_s2, h->sub_c, h->up_h, h->up_h, tmp);
    if (st == FD_OK) st = upload_f32(w->b_s2, h->b_s2, h->sub_c);
  }
  if (st == FD_OK && launch_state_reset(h->state, h->stream) != hipSuccess) st = FD_ERR_DEVICE;
  if (st == FD_OK && hipStreamSynchronize(h->stream) != hipSuccess) st = FD_ERR_DEVICE;
  if (st != FD_OK) {
    (void)hipFree(h->arena);
    delete h;
    return st;
  }
  *out = h;
  return FD_OK;
}

}  // extern "C"

namespace {

// This frame's temporal rotary table (pairs 0..11 of head_dim 64), in double
// on the host: the backbone's tokens sit at the frame's index t, sub-frame k
// of the tail at r_t t + k.  Keys are rotated once, at their own index; only
// index differences enter the scores, so this equals positions relative to
// the window.  Written to device memory by a launch of its own, ahead of the
// frame's other launches.
fd_status enqueue_rope_table(fd_handle* h) {
  if (!h->rope) return FD_OK;
  const fd_config& c = h->cfg;
  RopeTable rtab{};
  for (int k = 0; k < 12; ++k) {
    const double f = rope_freq(c.rope_theta, k, 24);
    const double a = (double)h->host_t * f;
    rtab.v[0][k] = make_float2((float)cos(a), (float)sin(a));
    for (int sf = 0; h->R && sf < c.out_t; ++sf) {
      const double as = ((double)h->host_t * c.out_t + sf) * f;
      rtab.v[1 + sf][k] = make_float2((float)cos(as), (float)sin(as));
    }
  }
  return run(h, FD_K_STATE, [&] { return launch_rope_table(h->rope_t, rtab, h->stream); });
}

// Every launch of one frame after the rotary table: ring bookkeeping,
// patchify, in-projection, the blocks, the output.  With via_state the
// latent and pixel buffers are taken from the ring state (set_io), so that
// the same launches serve every frame of a recorded graph; otherwise
// latent_dev and pixels_dev are passed directly.
fd_status enqueue_frame(fd_handle* h, const float* latent_dev, float* pixels_dev,
                        bool via_state) {
  const fd_config& c = h->cfg;
  const int D = h->D, F = h->F, M = h->m_rows, N = h->N, B = h->B;
  hipStream_t s = h->stream;

  // One pre-norm block over `rows` tokens per stream (the backbone's N, or
  // the tail's r_t N sub-frame tokens with sub_n = N), B streams stacked
  // row-wise, with its own ring of slot size ring_pad and `splits` attention
  // key splits.
  auto block = [&](const LayerPtrs& L, int rows_s, int ring_pad, int splits, int sub_n) -> fd_status {
    const int rows = B * rows_s;
    FD_TRY(run(h, FD_K_LN, [&] {
      return launch_layernorm(h->h, rows, D, L.ln1_g, L.ln1_b, c.ln_eps, h->rms, h->a, s);
    }));
    FD_TRY(run(h, FD_K_QKV, [&] {
      GemmArgs g{h->a, L.w_qkv, rows, h->qkv_n, D, epi_plain(L.b_qkv, nullptr, h->q, 0)};
      g.epi.ring_k = L.ring_k;
      g.epi.ring_vt = L.ring_vt;
      g.epi.state = h->state;
      g.epi.d_model = D;
      g.epi.head_dim = h->hd;
      g.epi.n_pad = ring_pad;
      g.epi.q_rows = h->q_rows;
      g.epi.kv_heads = h->kv_heads;
      g.epi.q_scale = h->q_scale;
      g.epi.kv_norm = h->kv_norm;
      g.epi.rope = h->rope;
      g.epi.norm_eps = c.ln_eps;
      g.epi.kn_g = L.kn_g;
      g.epi.vn_g = L.vn_g;
      g.epi.rope_h = h->rope_h;
      g.epi.rope_w = h->rope_w;
      g.epi.tok_w = h->tok_w;
      g.epi.sub_n = sub_n;
      g.epi.rows_s = rows_s;
      g.epi.heads = h->heads;
      g.epi.streams = B;
      // backbone rows use table row 0; sub-frame k of the tail uses row 1 + k
      g.epi.rope_t = h->rope_t ? h->rope_t + (sub_n ? 12 : 0) : nullptr;
      return launch_gemm(EPI_QKV, g, M, s);
    }));
    FD_TRY(run(h, FD_K_ATTN, [&] {
      AttnArgs a{h->q, L.ring_k, L.ring_vt, h->state, h->o, rows_s, ring_pad, h->q_rows,
                 B * h->heads, h->hd, h->W, h->q_scale, h->part_o, h->part_ml, splits,
                 B * h->kv_heads, h->heads};
      return launch_attention(a, s);
    }));
    FD_TRY(run(h, FD_K_OPROJ, [&] {
      GemmArgs g{h->o, L.w_o, rows, D, D, epi_plain(L.b_o, h->h, nullptr, D)};
      return launch_gemm(EPI_RESID, g, M, s);
    }));
    FD_TRY(run(h, FD_K_LN, [&] {
      return launch_layernorm(h->h, rows, D, L.ln2_g, L.ln2_b, c.ln_eps, h->rms, h->a, s);
    }));
    FD_TRY(run(h, FD_K_FC1, [&] {
      GemmArgs g{h->a, L.w_1, rows, F, D, epi_plain(L.b_1, nullptr, h->u, F)};
      return launch_gemm(EPI_GELU_BF16, g, M, s);
    }));
    FD_TRY(run(h, FD_K_FC2, [&] {
      GemmArgs g{h->u, L.w_2, rows, D, F, epi_plain(L.b_2, h->h, nullptr, D)};
      return launch_gemm(EPI_RESID, g, M, s);
    }));
    return FD_OK;
  };

  h->cur_layer = -1;
  FD_TRY(run(h, FD_K_STATE, [&] { return launch_frame_begin(h->state, h->W, s); }));
  const size_t latent_elems = (size_t)c.latent_c * c.latent_h * c.latent_w;
  for (int b = 0; b < B; ++b)
    FD_TRY(run(h, FD_K_PATCHIFY, [&] {
      const size_t off = b * latent_elems;
      return launch_patchify(via_state ? nullptr : latent_dev + off,
                             via_state ? h->state : nullptr, off, c.latent_c, c.latent_h,
                             c.latent_w, c.patch, h->k_in_pad,
                             h->x + (size_t)b * N * h->k_in_pad, s);
    }));
  FD_TRY(run(h, FD_K_INPROJ, [&] {
    GemmArgs g{h->x, h->w_in, B * N, D, h->k_in_pad, epi_plain(h->b_in, h->h, nullptr, D)};
    return launch_gemm(EPI_F32_BIAS, g, M, s);
  }));
  for (int l = 0; l < h->L; ++l) {
    h->cur_layer = l;
    FD_TRY(block(h->layers[l], N, h->n_pad, h->splits, 0));
  }
  h->cur_layer = -1;
  FD_TRY(run(h, FD_K_LN, [&] {
    return launch_layernorm(h->h, B * N, D, h->lnf_g, h->lnf_b, c.ln_eps, h->rms, h->a, s);
  }));
  // Pixel epilogue of the last GEMM: rows (stream, sub-frame, token) x
  // channels (tau, dy, dx, c).
  auto pixel_epi = [&](const float* bias, int rows_s, int sub_n) {
    EpiParams e = epi_plain(bias, pixels_dev, nullptr, 0);
    if (via_state) {
      e.state = h->state;
      e.out_from_state = 1;
    }
    e.tok_w = h->tok_w;
    e.patch_out = c.out_patch;
    e.out_c = c.out_c;
    e.out_t = c.out_t;
    e.pix_h = h->pix_h;
    e.pix_w = h->pix_w;
    e.sub_n = sub_n;
    e.rows_s = rows_s;
    return e;
  };
  if (h->R == 0) {
    FD_TRY(run(h, FD_K_UNPATCH, [&] {
      GemmArgs g{h->a, h->w_out, B * N, h->c_out, D, pixel_epi(h->b_out, N, 0)};
      return launch_gemm(EPI_PIXELS, g, M, s);
    }));
  } else {
    // Temporal-first upsampling tail ([FD] §3.4).  Step 1: the D -> r_t D
    // linear writes column block k of token n to row k N + n of the residual
    // stream (the backbone's H is dead once LNf has read it).
    FD_TRY(run(h, FD_K_TEMPORAL, [&] {
      GemmArgs g{h->a, h->w_tu, B * N, c.out_t * D, D, epi_plain(h->b_tu, h->h, nullptr, D)};
      g.epi.d_model = D;
      g.epi.sub_n = N;
      g.epi.out_t = c.out_t;
      return launch_gemm(EPI_SUBFRAMES, g, M, s);
    }));
    // Step 2: refinement blocks over the r_t N sub-frame tokens.
    for (int r = 0; r < h->R; ++r) {
      h->cur_layer = h->L + r;
      FD_TRY(block(h->rlayers[r], h->N4, h->n4_pad, h->splits_r, N));
    }
    h->cur_layer = -1;
    // Step 3: norm, D -> Hs GELU, Hs -> r_s^2 C with the PixelShuffle store.
    const int rows4 = B * h->N4;
    FD_TRY(run(h, FD_K_LN, [&] {
      return launch_layernorm(h->h, rows4, D, h->lnr_g, h->lnr_b, c.ln_eps, h->rms, h->a, s);
    }));
    FD_TRY(run(h, FD_K_SPATIAL, [&] {
      GemmArgs g{h->a, h->w_s1, rows4, h->up_h, D, epi_plain(h->b_s1, nullptr, h->u, h->up_h)};
      return launch_gemm(EPI_GELU_BF16, g, M, s);
    }));
    FD_TRY(run(h, FD_K_UNPATCH, [&] {
      GemmArgs g{h->u, h->w_s2, rows4, h->sub_c, h->up_h, pixel_epi(h->b_s2, h->N4, N)};
      return launch_gemm(EPI_PIXELS, g, M, s);
    }));
  }
  return FD_OK;
}

void drop_graph(fd_handle* h) {
  if (h->graph_exec) (void)hipGraphExecDestroy(h->graph_exec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  h->graph_exec = nullptr;
  h->graph = nullptr;
}

}  // namespace

extern "C" {

fd_status fd_decode_frame(fd_handle* h, const float* latent_dev, float* pixels_dev) {
  if (!h || !latent_dev || !pixels_dev) return FD_ERR_INVALID_ARG;
  if (((uintptr_t)latent_dev & 3) || ((uintptr_t)pixels_dev & 15)) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  FD_TRY(enqueue_rope_table(h));
  if (h->graph_exec) {
    FD_TRY(run(h, FD_K_STATE,
               [&] { return launch_set_io(h->state, latent_dev, pixels_dev, h->stream); }));
    FD_TRY(run(h, FD_K_STATE, [&] { return hipGraphLaunch(h->graph_exec, h->stream); }));
  } else {
    FD_TRY(enqueue_frame(h, latent_dev, pixels_dev, false));
  }
  ++h->host_t;
  return FD_OK;
}

fd_status fd_graph_enable(fd_handle* h, int enable) {
  if (!h) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  if (h->graph_exec) {
    // A replay may still be running: let it finish before the graph goes.
    if (hipStreamSynchronize(h->stream) != hipSuccess) {
      h->broken = true;
      return FD_ERR_DEVICE;
    }
    drop_graph(h);
  }
  if (!enable) return FD_OK;
  if (h->profiling) return FD_ERR_INVALID_ARG;
  // Capture is not possible on the legacy default stream.
  if (!h->stream) return FD_ERR_UNSUPPORTED;
  if (hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipGetLastError();
    return FD_ERR_UNSUPPORTED;
  }
  const fd_status st = enqueue_frame(h, nullptr, nullptr, true);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(h->stream, &g);
  if (st != FD_OK || ec != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    // An injected launch failure has broken the handle (FD_ERR_DEVICE);
    // otherwise the handle stays as it was, without a graph.
    return st != FD_OK ? st : FD_ERR_UNSUPPORTED;
  }
  if (hipGraphInstantiate(&h->graph_exec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    h->graph_exec = nullptr;
    return FD_ERR_UNSUPPORTED;
  }
  h->graph = g;
  return FD_OK;
}

fd_status fd_reset(fd_handle* h) {
  if (!h) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  const fd_status st = run(h, FD_K_STATE, [&] { return launch_state_reset(h->state, h->stream); });
  if (st == FD_OK) h->host_t = 0;
  return st;
}

void fd_destroy(fd_handle* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->stream);
  drop_graph(h);
  for (hipEvent_t e : h->event_pool) (void)hipEventDestroy(e);
  if (h->arena) (void)hipFree(h->arena);
  delete h;
}

fd_status fd_query(const fd_handle* h, fd_info* info) {
  if (!h || !info) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  DeviceState ds;
  if (hipStreamSynchronize(h->stream) != hipSuccess ||
      hipMemcpy(&ds, h->state, sizeof ds, hipMemcpyDeviceToHost) != hipSuccess) {
    const_cast<fd_handle*>(h)->broken = true;
    return FD_ERR_DEVICE;
  }
  memset(info, 0, sizeof *info);
  info->frames_decoded = ds.frames_done;
  info->n_valid = ds.frames_done == 0 ? 0 : ds.n_valid;
  info->window = h->W;
  for (int i = 0; i < FD_MAX_WINDOW; ++i) info->slot_frame[i] = i < h->W ? ds.slot_frame[i] : -1;
  info->n_tokens = h->N;
  info->n_tokens_pad = h->n_pad;
  info->arena_bytes = h->arena_bytes;
  info->weight_bytes = h->weight_bytes;
  info->ring_bytes = h->ring_bytes;
  info->workspace_bytes = h->ws_bytes;
  return FD_OK;
}

fd_status fd_debug_read_kv(const fd_handle* h, int layer, int slot, int kv,
                           uint16_t* host_bf16, size_t count) {
  if (!h || !host_bf16) return FD_ERR_INVALID_ARG;
  if (layer < 0 || layer >= h->L + h->R || slot < 0 || slot >= h->W || (kv != 0 && kv != 1))
    return FD_ERR_INVALID_ARG;
  const bool refine = layer >= h->L;
  const int N = refine ? h->N4 : h->N, np = refine ? h->n4_pad : h->n_pad, hd = h->hd;
  const int G = h->B * h->kv_heads;          // every stream's KV heads
  if (count != (size_t)G * N * hd) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  const size_t slot_elems = (size_t)G * np * hd;
  const LayerPtrs& L = refine ? h->rlayers[layer - h->L] : h->layers[layer];
  const uint16_t* src = (kv == 0 ? L.ring_k : L.ring_vt) + slot * slot_elems;
  std::vector<uint16_t> tmp(slot_elems);
  if (hipStreamSynchronize(h->stream) != hipSuccess ||
      hipMemcpy(tmp.data(), src, slot_elems * 2, hipMemcpyDeviceToHost) != hipSuccess) {
    const_cast<fd_handle*>(h)->broken = true;
    return FD_ERR_DEVICE;
  }
  for (int hh = 0; hh < G; ++hh)
    for (int n = 0; n < N; ++n)
      for (int d = 0; d < hd; ++d)
        host_bf16[((size_t)hh * N + n) * hd + d] =
            kv == 0 ? tmp[((size_t)hh * np + n) * hd + d]
                    : tmp[((size_t)hh * hd + d) * np + vt_perm(n)];
  return FD_OK;
}

fd_status fd_debug_read_ring(const fd_handle* h, int layer, int slot, int kv,
                             uint16_t* host_bf16, size_t count) {
  if (!h || !host_bf16) return FD_ERR_INVALID_ARG;
  if (layer < 0 || layer >= h->L + h->R || slot < 0 || slot >= h->W || (kv != 0 && kv != 1))
    return FD_ERR_INVALID_ARG;
  const bool refine = layer >= h->L;
  const int np = refine ? h->n4_pad : h->n_pad;
  const size_t slot_elems = (size_t)h->B * h->kv_heads * np * h->hd;
  if (count != slot_elems) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  const LayerPtrs& L = refine ? h->rlayers[layer - h->L] : h->layers[layer];
  const uint16_t* src = (kv == 0 ? L.ring_k : L.ring_vt) + slot * slot_elems;
  if (hipStreamSynchronize(h->stream) != hipSuccess ||
      hipMemcpy(host_bf16, src, slot_elems * 2, hipMemcpyDeviceToHost) != hipSuccess) {
    const_cast<fd_handle*>(h)->broken = true;
    return FD_ERR_DEVICE;
  }
  return FD_OK;
}

fd_status fd_debug_poison_ring(fd_handle* h) {
  if (!h) return FD_ERR_INVALID_ARG;
  if (h->broken) return FD_ERR_STATE;
  const int heads = h->W * h->B * h->kv_heads;
  for (const LayerPtrs& l : h->layers)
    FD_TRY(run(h, FD_K_STATE, [&] {
      return launch_poison_ring(l.ring_k, l.ring_vt, heads, h->N, h->n_pad, h->hd, h->stream);
    }));
  for (const LayerPtrs& l : h->rlayers)
    FD_TRY(run(h, FD_K_STATE, [&] {
      return launch_poison_ring(l.ring_k, l.ring_vt, heads, h->N4, h->n4_pad, h->hd, h->stream);
    }));
  return FD_OK;
}

fd_status fd_debug_fail_after(fd_handle* h, int64_t launches) {
  if (!h) return FD_ERR_INVALID_ARG;
  h->fail_after = launches < 0 ? -1 : launches;
  return FD_OK;
}

// ----------------------------------------------------------------- profiling
fd_status fd_profile_enable(fd_handle* h, int enable) {
  if (!h) return FD_ERR_INVALID_ARG;
  // A replayed graph makes no per-launch event records.
  if (enable && h->graph_exec) return FD_ERR_INVALID_ARG;
  h->profiling = enable != 0;
  return FD_OK;
}

fd_status fd_profile_filter(fd_handle* h, uint32_t kind_mask, int layer) {
  if (!h || layer < -1) return FD_ERR_INVALID_ARG;
  h->prof_mask = kind_mask;
  h->prof_layer = layer;
  return FD_OK;
}

fd_status fd_profile_read(fd_handle* h, double* ms, int64_t* launches, int n_kinds) {
  if (!h || !ms || !launches || n_kinds < FD_K_COUNT) return FD_ERR_INVALID_ARG;
  if (hipStreamSynchronize(h->stream) != hipSuccess) {
    h->broken = true;
    return FD_ERR_DEVICE;
  }
  for (int k = 0; k < n_kinds; ++k) { ms[k] = 0.0; launches[k] = 0; }
  for (const auto& r : h->recs) {
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess) {
      ms[r.kind] += t;
      launches[r.kind] += 1;
    }
  }
  h->recs.clear();
  h->pool_used = 0;
  return FD_OK;
}

// ------------------------------------------------- per-step test entry points
fd_status fdk_gemm(int epi, const uint16_t* a, const uint16_t* b, const float* bias,
                   void* out, int m, int m_rows_alloc, int n, int k, void* stream) {
  if (!a || !b || !bias || !out || m < 0 || n <= 0 || k <= 0) return FD_ERR_INVALID_ARG;
  if (epi != EPI_F32_BIAS && epi != EPI_RESID && epi != EPI_GELU_BF16) return FD_ERR_INVALID_ARG;
  if (k % 64 || n % 64 || m_rows_alloc % 64 || m_rows_alloc < m) return FD_ERR_UNSUPPORTED;
  GemmArgs g{a, b, m, n, k,
             epi == EPI_GELU_BF16 ? epi_plain(bias, nullptr, (uint16_t*)out, n)
                                  : epi_plain(bias, (float*)out, nullptr, n)};
  return launch_gemm(epi, g, m_rows_alloc, (hipStream_t)stream) == hipSuccess ? FD_OK
                                                                             : FD_ERR_DEVICE;
}

fd_status fdk_layernorm(const float* x, int m, int d, const float* g, const float* b,
                        float eps, int rms, uint16_t* out, void* stream) {
  if (!x || !g || (!b && !rms) || !out || m < 0 || (rms != 0 && rms != 1))
    return FD_ERR_INVALID_ARG;
  if (!ln_dim_ok(d)) return FD_ERR_UNSUPPORTED;
  return launch_layernorm(x, m, d, g, b, eps, rms, out, (hipStream_t)stream) == hipSuccess
             ? FD_OK : FD_ERR_DEVICE;
}

}  // extern "C"
