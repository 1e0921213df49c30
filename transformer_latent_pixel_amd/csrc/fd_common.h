// Shared device types and helpers of the gfx950 decode path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashdec.h"

namespace fd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin

// Ring bookkeeping, resident in device memory so that every kernel of a frame
// reads it instead of taking it as a launch argument.
struct DeviceState {
  int frames_done;                // frames decoded so far = t of the next frame
  int t;                          // frame being decoded
  int write_slot;                 // t mod W
  int n_valid;                    // min(t + 1, W)
  int slot_frame[FD_MAX_WINDOW];  // frame held by each slot, -1 if empty
  int chrono_slot[FD_MAX_WINDOW]; // valid slots, oldest frame first
  // The caller's buffers of the frame being decoded, for launches that take
  // them from here instead of as arguments (a replayed graph's launches keep
  // the arguments they were recorded with).
  const float* latent;
  float* pixels;
};

// Round-to-nearest-even float -> bf16 bits (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// fp16 (IEEE binary16) bits, round to nearest even, and back.
__device__ __forceinline__ uint32_t f2h2(float lo, float hi) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Values are stored in the ring with bits 2 and 3 of the token index swapped
// inside every 32-token group: that puts the 8 keys one lane needs as an MFMA
// operand (tokens 4h..4h+3 and 4h+8..4h+11 of a 16-key chunk) side by side.
__host__ __device__ __forceinline__ int vt_perm(int n) {
  return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

// Epilogue kinds of the bf16 GEMM.
enum Epilogue : int {
  EPI_F32_BIAS = 0,   // out_f32[m][n]  = acc + bias[n]
  EPI_RESID = 1,      // out_f32[m][n] += acc + bias[n]
  EPI_GELU_BF16 = 2,  // out_bf16[m][n] = GELU(acc + bias[n])
  EPI_QKV = 3,        // scatter to Q buffer and the K / V^T ring slot
  EPI_PIXELS = 4,     // pixel-shuffle store of acc + bias[n]
  EPI_SUBFRAMES = 5   // out_f32[(n / d_model) sub_n + m][n % d_model] = acc + bias[n]
};

struct EpiParams {
  const float* bias;
  float* out_f32;      // EPI_F32_BIAS, EPI_RESID, EPI_PIXELS
  uint16_t* out_bf16;  // EPI_GELU_BF16, EPI_QKV (Q)
  int ldo;             // row stride of out_f32 / out_bf16 (elements)
  // EPI_QKV: columns [0, d_model) are Q heads, then kv_heads K heads, then
  // kv_heads V heads (head_dim columns each).
  uint16_t* ring_k;    // this block's K ring: [W][kv_heads][n_pad][hd]
  uint16_t* ring_vt;   // this block's V^T ring: [W][kv_heads][hd][n_pad] (vt_perm'd)
  const DeviceState* state;
  int d_model, head_dim, n_pad, q_rows;  // q buffer: [heads][q_rows][hd]
  int kv_heads;
  float q_scale;       // folded into Q before rounding
  // The paper's block (head_dim 64 only): KV-norm gains and eps; rotary
  // cos/sin per pair: temporal pairs 0..11 from rope_t[sub-frame of the
  // row][pair] (device memory, written at the start of every frame), row
  // pairs 12..21 from rope_h[token row], column pairs 22..31 from
  // rope_w[token column].
  int kv_norm, rope;
  float norm_eps;
  const float* kn_g;
  const float* vn_g;
  const float2* rope_t;   // [sub-frame][12]
  const float2* rope_h;   // [tok_h][10]
  const float2* rope_w;   // [tok_w][10]
  // EPI_PIXELS (tok_w also for the rotary positions); out_from_state: the
  // pixel buffer is state->pixels, not out_f32
  int tok_w, patch_out, out_c, pix_h, pix_w, out_t;
  int out_from_state;
  // Streams and sub-frames.  Row m belongs to stream m / rows_s (rows_s =
  // the token rows of one stream, 0 = one stream) and is row r = m % rows_s
  // of it.  In the upsampling tail row r is spatial token r % sub_n of
  // sub-frame r / sub_n (rotary temporal table, pixel frame); sub_n = 0:
  // every row is spatial token r of sub-frame 0.  EPI_SUBFRAMES: rows_s =
  // sub_n = N, and token n of stream b goes to rows (b out_t + k) N + n.
  // EPI_QKV with streams: Q head j of stream b is Q head b heads + j; KV
  // head g of stream b is ring head b kv_heads + g (kv_heads per stream).
  int sub_n, rows_s, heads, streams;
};

struct GemmArgs {
  const uint16_t* a;   // [m_rows][k] bf16, m_rows a multiple of the tile M
  const uint16_t* b;   // [n][k] bf16 (Linear weight, row-major [out][in])
  int m;               // rows to store (valid rows)
  int n, k;
  EpiParams epi;
};

// Launchers (enqueue only; return hipError_t of the launch).
hipError_t launch_gemm(int epi, const GemmArgs& args, int m_rows_alloc,
                       hipStream_t s);
// rms = 0: LayerNorm (b is the shift); rms = 1: RMSNorm (b unused).
hipError_t launch_layernorm(const float* h, int m, int d, const float* g,
                            const float* b, float eps, int rms, uint16_t* out,
                            hipStream_t s);
// Patchify the latent z, or with io the latent io->latent + z_off.
hipError_t launch_patchify(const float* z, const DeviceState* io, size_t z_off, int c, int hl,
                           int wl, int p, int k_pad, uint16_t* x, hipStream_t s);
hipError_t launch_set_io(DeviceState* st, const float* latent, float* pixels, hipStream_t s);

// Temporal rotary cos/sin of one frame, computed on the host: row 0 for the
// backbone (the frame's index t), rows 1 .. r_t for the sub-frames of the
// upsampling tail (r_t t + k).  Copied into device memory by a one-thread
// kernel at the start of the frame.
constexpr int kRopeRows = FD_MAX_SUBFRAMES + 1;
struct RopeTable {
  float2 v[kRopeRows][12];
};
hipError_t launch_rope_table(float2* dst, const RopeTable& tab, hipStream_t s);

struct AttnArgs {
  const uint16_t* q;        // [heads][q_rows][hd], pre-scaled by q_scale
  const uint16_t* ring_k;   // [W][kv_heads][n_pad][hd]
  const uint16_t* ring_vt;  // [W][kv_heads][hd][n_pad], vt_perm'd token order
  const DeviceState* state;
  uint16_t* o;              // [n][heads*hd]
  int n, n_pad, q_rows, heads, head_dim, window;
  float q_scale;            // scale already folded into q (for the generic path)
  // Key splits (attention_splits): with splits > 1 each split writes its
  // normalised partial output and (max, sum, scale) here, and a combine pass
  // produces o.  part_o: fp16 bits [splits][n][heads*hd] (a normalised
  // partial is a convex combination of V rows; fp16 keeps it to 2^-11,
  // finer than the bf16 rounding of the merged output), divided by the
  // scale, a power of two that is 1 unless the partial reaches 2^15;
  // part_ml: fp32 [splits][heads][n][4] = (max, sum, scale, 0).
  uint16_t* part_o;
  float* part_ml;
  int splits;
  int kv_heads;             // query head j reads KV head j * kv_heads / heads
  // Streams: heads and kv_heads count every stream's heads (stream b owns
  // heads b H .. b H + H - 1 and KV heads b G ..); O holds o_heads heads per
  // row and stream b's queries at rows b n .. b n + n - 1.  0 = heads.
  int o_heads;
};
// Number of key splits (1..4) for the attention of heads x n queries, from
// a cost model of workgroup rounds on 256 CUs (independent of the window).
int attention_splits(int heads, int n, int head_dim);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

hipError_t launch_frame_begin(DeviceState* st, int window, hipStream_t s);
// Fill the token rows (< n) of every ring slot with bf16 NaN, K [heads][n_pad][hd]
// and V^T [heads][hd][n_pad] (vt_perm'd); padding rows are left as they are.
hipError_t launch_poison_ring(uint16_t* ring_k, uint16_t* ring_vt, int heads, int n,
                              int n_pad, int hd, hipStream_t s);
hipError_t launch_state_reset(DeviceState* st, hipStream_t s);

}  // namespace fd
