// bf16 x bf16 -> fp32 GEMM on gfx950 matrix cores, with the decode step's
// fused epilogues: C[m][n] = sum_k A[m][k] * B[n][k] (+ bias, then one of
// store fp32 / residual add / GELU to bf16 / Q-K-V scatter / pixel shuffle).
//
// Design (gfx950):
//  * v_mfma_f32_32x32x16_bf16; each wave owns a (TM*32) x (TN*32) sub-tile.
//  * K steps of 32 stream through a ring of 3 or 4 LDS stages filled by
//    direct global->LDS loads (global_load_lds_dwordx4), 2 or 3 steps ahead
//    of the MFMAs, with one workgroup barrier per step and no staging
//    registers.
//  * LDS rows are 4 chunks of 16 bytes; chunk c of row r is stored at
//    c ^ ((r >> 2) & 3).  A 16-byte LDS read serves 16 lanes per cycle over
//    64 banks (16 groups of 16 bytes); the 16 consecutive rows those lanes
//    read at one chunk then fall on 16 distinct groups.
//  * Tiles are dealt to the 8 XCDs in contiguous runs (workgroup i runs on
//    XCD i % 8), and inside a run in column-major groups of 8 tile rows, so
//    that the tiles resident on one XCD share A rows and B columns in its L2.
//  * The bf16 row outputs (GELU, and Q and K of the QKV scatter) are staged
//    per 32-row block in a wave-private slice of the idle B stages and
//    stored as whole 128-byte rows; fp32 outputs are stored directly.
#include "fd_common.h"

namespace fd {
namespace {

// GELU(x) = x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), branch-free.  erf by
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// for z >= 0, erf(z) = 1 - (a1 t + ... + a5 t^5) exp(-z^2), t = 1/(1 + p z),
// |error| <= 1.5e-7.  With z = |x|/sqrt 2 and q = (a1 t + ... + a5 t^5)
// exp(-z^2), 1 + erf(x/sqrt 2) is 2 - q for x >= 0 and q for x < 0, so
// GELU(x) = max(x, 0) - 0.5 |x| q for either sign (no cancellation for
// negative x).  The 0.5 is folded into the a_i, 1/sqrt 2 into p, and
// exp(-z^2) = 2^(x * (x * -log2(e) / 2)).
__device__ __forceinline__ float gelu_erf(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, ax, 1.0f));
  float p = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  p = fmaf(t, p, 0.5f * 1.421413741f);
  p = fmaf(t, p, 0.5f * -0.284496736f);
  p = fmaf(t, p, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(x * (x * (-0.5f * 1.4426950408889634f)));
  const float hq = p * t * e;                  // 0.5 q
  return fmaf(-ax, hq, fmaxf(x, 0.0f));
}

// QKV scatter of 4 consecutive columns n..n+3 of row m of stream b (they
// lie in one head).  Columns [0, d_model) are the Q heads, then kv_heads K
// heads, then kv_heads V heads.  Q goes to [stream head][q_rows][hd] scaled
// by q_scale, K to ring slot [stream kv head][n_pad][hd], V transposed to
// [stream kv head][hd][n_pad] with the token order vt_perm'd.
__device__ __forceinline__ void qkv_store4(const EpiParams& e, int b, int m, int n,
                                           const floatx4& v, int write_slot) {
  const int hd = e.head_dim, nq = e.d_model, nk = e.kv_heads * hd;
  const int which = n < nq ? 0 : (n < nq + nk ? 1 : 2);
  const int r = n - (which == 0 ? 0 : (which == 1 ? nq : nq + nk));
  const int head = r / hd, d = r - head * hd;
  // KV head of this stream within the ring slot, and Q head of this stream.
  const int ns = e.streams > 0 ? e.streams : 1;
  const size_t kvh = ((size_t)write_slot * ns + b) * e.kv_heads + head;
  if (which == 2) {
    uint16_t* vt = e.ring_vt + kvh * (size_t)hd * e.n_pad +
                   (size_t)d * e.n_pad + vt_perm(m);
    vt[0] = f2bf(v[0]);
    vt[e.n_pad] = f2bf(v[1]);
    vt[2 * (size_t)e.n_pad] = f2bf(v[2]);
    vt[3 * (size_t)e.n_pad] = f2bf(v[3]);
  } else {
    const float sc = which == 0 ? e.q_scale : 1.0f;
    uint2 w;
    w.x = f2bf2(v[0] * sc, v[1] * sc);
    w.y = f2bf2(v[2] * sc, v[3] * sc);
    uint16_t* dst = which == 0
        ? e.out_bf16 + ((size_t)(b * e.heads + head) * e.q_rows + m) * hd + d
        : e.ring_k + kvh * (size_t)e.n_pad * hd + (size_t)m * hd + d;
    *reinterpret_cast<uint2*>(dst) = w;
  }
}

// Rotary cos/sin of pair p (0..31) of a head_dim-64 head for the token at
// row ti, column tj of sub-frame sf: temporal pairs 0..11 from that
// sub-frame's table, row pairs 12..21 and column pairs 22..31 from the
// per-token tables.
__device__ __forceinline__ float2 rope_cs(const EpiParams& e, int p, int ti, int tj, int sf) {
  if (p < 12) return e.rope_t[sf * 12 + p];
  if (p < 22) return e.rope_h[ti * 10 + (p - 12)];
  return e.rope_w[tj * 10 + (p - 22)];
}

// Epilogue stores.  The MFMA is issued as D = W Act^T, so a lane owns one
// output row m and holds 4 consecutive output columns n..n+3 (n % 4 == 0):
// fp32 results leave as one 16-byte store, bf16 results as one 8-byte store.
// b: the bias of columns n..n+3; h (EPI_RESID): the residual at (m, n..n+3),
// loaded by the caller before any store of the tile.
template <int EPI>
__device__ __forceinline__ void epi_store4(const EpiParams& e, int m, int n,
                                           floatx4 v, int write_slot, float4 b, float4 h) {
  v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
  if constexpr (EPI == EPI_F32_BIAS) {
    *reinterpret_cast<float4*>(e.out_f32 + (size_t)m * e.ldo + n) =
        make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (EPI == EPI_RESID) {
    h.x += v[0]; h.y += v[1]; h.z += v[2]; h.w += v[3];
    *reinterpret_cast<float4*>(e.out_f32 + (size_t)m * e.ldo + n) = h;
  } else if constexpr (EPI == EPI_GELU_BF16) {
    uint2 w;
    w.x = f2bf2(gelu_erf(v[0]), gelu_erf(v[1]));
    w.y = f2bf2(gelu_erf(v[2]), gelu_erf(v[3]));
    *reinterpret_cast<uint2*>(e.out_bf16 + (size_t)m * e.ldo + n) = w;
  } else if constexpr (EPI == EPI_QKV) {
    const int b = e.rows_s ? m / e.rows_s : 0;
    qkv_store4(e, b, m - b * e.rows_s, n, v, write_slot);
  } else if constexpr (EPI == EPI_PIXELS) {
    // channel n = ((tau P + dy) P + dx) C + c -> pixel[tau][i P + dy][j P + dx][c];
    // n .. n+3 stay inside one (tau, dy) run of P*C channels (P*C % 4 == 0).
    // With sub_n, row m is token m % sub_n of pixel frame m / sub_n.
    const int P = e.patch_out, C = e.out_c;
    const int per_t = P * P * C;
    const int b = e.rows_s ? m / e.rows_s : 0;
    const int rr = m - b * e.rows_s;
    const int sf = e.sub_n ? rr / e.sub_n : 0;
    const int mt = rr - sf * e.sub_n;
    const int tau = n / per_t;
    int r = n - tau * per_t;
    const int dy = r / (P * C);
    r -= dy * (P * C);                                   // dx * C + c
    const int i = mt / e.tok_w, j = mt - i * e.tok_w;
    const size_t off = (((size_t)(b * e.out_t + tau + sf) * e.pix_h + (size_t)i * P + dy) *
                            e.pix_w + (size_t)j * P) * C + r;
    *reinterpret_cast<float4*>(e.out_f32 + off) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (EPI == EPI_SUBFRAMES) {
    // column block k = n / d_model of token t of stream b (row m = b sub_n
    // + t) becomes row (b out_t + k) sub_n + t (n .. n+3 stay in one block:
    // d_model % 4 == 0).
    const int k = n / e.d_model, d = n - k * e.d_model;
    const int b = m / e.sub_n, t = m - b * e.sub_n;
    *reinterpret_cast<float4*>(e.out_f32 +
                               ((size_t)(b * e.out_t + k) * e.sub_n + t) * e.d_model + d) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (other counters untouched; gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS stage ring.  Each wave has already waited
// for its own loads of the stage about to be read (wait_vmcnt), so the
// barrier only has to order waves; __syncthreads() would add a release
// fence that drains every load in flight, including the later stages.
// The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds + 16 i (lds must be wave-uniform).  Kept in
// a __device__ function so the builtin is only seen by the device pass.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds,
                                   16, 0, 0);
}

// LDS stage layout: BM + BN rows of BK = 32 bf16 (64 bytes = 4 chunks of 16
// bytes); chunk c of row r sits at c ^ ((r >> 2) & 3), so 16 consecutive rows
// read at the same chunk hit 16 distinct 16-byte bank groups (rows r and
// r + 4k share (4 r) mod 16 and differ in the XOR key).
__device__ __forceinline__ int swz32(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Block tile BM x BN, waves WAVES_M x WAVES_N; each wave (BM/WAVES_M) x (BN/WAVES_N).
// K steps of 32 stream through a ring of STAGES (3 or 4) LDS stages filled by
// direct global->LDS loads (global_load_lds_dwordx4), STAGES-1 steps ahead of
// the MFMAs.  MINB workgroups are meant to share a CU (registers are capped
// to fit), so that one workgroup's epilogue overlaps another's main loop.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int MINB, int EPI>
__global__ __launch_bounds__(kWave * WAVES_M * WAVES_N, MINB)
void gemm_bf16_kernel(const GemmArgs args_in) {
  const GemmArgs args = args_in;
  static_assert(STAGES == 3 || STAGES == 4, "ring depth");
  constexpr int BK32 = 32;
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int LOADS = ROWS / 16;            // 1-KB wave loads per stage
  static_assert(LOADS % NWAVES == 0, "stage loads must divide over waves");
  constexpr int CPT = LOADS / NWAVES;         // loads per wave per stage
  // One array per stage and operand: distinct LDS objects let the compiler
  // see that reads of one stage never alias loads still landing in another.
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[BM * 64], sb0[BN * 64];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[BM * 64], sb1[BN * 64];
  __shared__ __attribute__((aligned(1024))) uint8_t sa2[BM * 64], sb2[BN * 64];
  __shared__ __attribute__((aligned(1024))) uint8_t sa3[STAGES == 4 ? BM * 64 : 16],
      sb3[STAGES == 4 ? BN * 64 : 16];

  const int K = args.k;
  const int tiles_m = (args.m + BM - 1) / BM;
  const int tiles_n = args.n / BN;
  const int T = tiles_m * tiles_n;

  // XCD-aware remap: the run of logical tiles [x*per + min(x,rem), ...) goes
  // to XCD x; column-major inside groups of 8 tile rows.
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + idx;
  constexpr int GM = 8;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in_g = logical - group * GM * tiles_n;
  const int tm = first_m + in_g % gsize;
  const int tn = in_g / gsize;

  const int tid = threadIdx.x;
  // The wave index is uniform; readfirstlane lets the compiler keep
  // everything derived from it in scalar registers.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int r32 = lane & 31, half = lane >> 5;

  const uint16_t* gA = args.a + (size_t)tm * BM * K;
  const uint16_t* gB = args.b + (size_t)tn * BN * K;

  // Load j of this wave fills stage rows [row0, row0 + 16) (rows < BM are A
  // rows, the rest B rows): lane i writes LDS bytes row0*64 + 16 i, i.e. row
  // row0 + i/4, physical chunk i%4, so it fetches logical chunk
  // (i%4) ^ ((row >> 2) & 3) of that row.
  // Addressing: a wave-uniform base (A or B block, advanced by the K step)
  // plus a per-lane 32-bit byte offset held in a register for the whole
  // loop, so the load uses the SGPR-base form and its VGPR operand is never
  // overwritten while the load is in flight.
  const uint8_t* gbase[CPT];
  uint32_t voff[CPT];
  int lds_off[CPT];
  bool in_a[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int row0 = (wave * CPT + j) * 16;
    const int row = row0 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    in_a[j] = row0 < BM;
    gbase[j] = reinterpret_cast<const uint8_t*>(in_a[j] ? gA : gB);
    voff[j] = (uint32_t)(((in_a[j] ? row : row - BM) * K + c * 8) * 2);
    lds_off[j] = (in_a[j] ? row0 : row0 - BM) * 64;
  }
  // The empty asm marks voff as redefined at each use, which stops the
  // compiler from hoisting gbase + voff into a 64-bit temporary.
#define FD_GEMM_ISSUE(SA_, SB_, KT_)                                               \
  _Pragma("unroll") for (int j_ = 0; j_ < CPT; ++j_) {                            \
    asm volatile("" : "+v"(voff[j_]));                                             \
    dma16(gbase[j_] + (size_t)(KT_) * (BK32 * 2) + voff[j_],                       \
          (in_a[j_] ? (SA_) : (SB_)) + lds_off[j_]);                               \
  }

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

#define FD_GEMM_COMPUTE(SA_, SB_)                                                   \
  {                                                                                 \
    const uint8_t* sA = (SA_);                                                      \
    const uint8_t* sB = (SB_);                                                      \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                              \
      const int chunk = kk * 2 + half;                                              \
      bf16x8 af[TM], bfr[TN];                                                       \
      _Pragma("unroll") for (int i = 0; i < TM; ++i) af[i] =                        \
          *reinterpret_cast<const bf16x8*>(sA + swz32(wm * WM + i * 32 + r32, chunk)); \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) bfr[j] =                       \
          *reinterpret_cast<const bf16x8*>(sB + swz32(wn * WN + j * 32 + r32, chunk)); \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i],        \
                                                              acc[i][j], 0, 0, 0);  \
    }                                                                               \
  }

  const int KT = K / BK32;
  // Prologue: steps 0..STAGES-2 in flight (steps past the end re-fetch the
  // last one, keeping the per-wave count of loads in flight uniform).
  FD_GEMM_ISSUE(sa0, sb0, 0)
  FD_GEMM_ISSUE(sa1, sb1, 1 < KT ? 1 : KT - 1)
  if constexpr (STAGES == 4) FD_GEMM_ISSUE(sa2, sb2, 2 < KT ? 2 : KT - 1)
  // Step kt: wait for its stage (STAGES-2 later stages may stay in flight),
  // one barrier (everyone's data landed, everyone is done with step kt-1),
  // refill the stage step kt-1 used with step kt+STAGES-1, then the MFMAs.
#define FD_GEMM_STEP(CA_, CB_, NA_, NB_, KT_)                                       \
  {                                                                                 \
    wait_vmcnt<(STAGES - 2) * CPT>();                                               \
    stage_barrier();                                                                \
    FD_GEMM_ISSUE(NA_, NB_, (KT_) + STAGES - 1 < KT ? (KT_) + STAGES - 1 : KT - 1)   \
    FD_GEMM_COMPUTE(CA_, CB_)                                                       \
  }
  if constexpr (STAGES == 4) {
    for (int kt = 0; kt < KT; kt += 4) {
      FD_GEMM_STEP(sa0, sb0, sa3, sb3, kt)
      if (kt + 1 < KT) FD_GEMM_STEP(sa1, sb1, sa0, sb0, kt + 1)
      if (kt + 2 < KT) FD_GEMM_STEP(sa2, sb2, sa1, sb1, kt + 2)
      if (kt + 3 < KT) FD_GEMM_STEP(sa3, sb3, sa2, sb2, kt + 3)
    }
  } else {
    for (int kt = 0; kt < KT; kt += 3) {
      FD_GEMM_STEP(sa0, sb0, sa2, sb2, kt)
      if (kt + 1 < KT) FD_GEMM_STEP(sa1, sb1, sa0, sb0, kt + 1)
      if (kt + 2 < KT) FD_GEMM_STEP(sa2, sb2, sa1, sb1, kt + 2)
    }
  }
  wait_vmcnt<0>();
#undef FD_GEMM_STEP
#undef FD_GEMM_COMPUTE
#undef FD_GEMM_ISSUE

  EpiParams epi = args.epi;
  if constexpr (EPI == EPI_PIXELS)
    if (epi.out_from_state) epi.out_f32 = epi.state->pixels;
  int write_slot = 0;
  if constexpr (EPI == EPI_QKV) write_slot = epi.state->write_slot;

  // acc[i][j] holds D = W Act^T for m-block i and n-block j: output row
  // m = lane % 32 of the block, output columns 8 * g + 4 * (lane / 32) + 0..3
  // from registers 4 g .. 4 g + 3.
  const int m0 = tm * BM + wm * WM;
  const int n0 = tn * BN + wn * WN;
  // The epilogue's loads (bias, residual) are issued ahead of the stores
  // they feed: the compiler cannot move a load above a store it may alias,
  // so loads interleaved with the stores would each wait a full memory
  // latency.  Most epilogues load the bias of the whole wave tile first; the
  // residual epilogue loads bias and residual per 32 x 32 block (one wait per
  // block), which keeps its registers within 128, so that two workgroups can
  // share a CU when a GEMM needs more than one round of tiles.  (The
  // per-head path of the QKV epilogue keeps its own loads: it stores nothing
  // before them, and preloading there measured slower.)
  float4 bv[EPI == EPI_RESID ? 1 : TN][4];
  auto load_bias = [&]() {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bv[j][g] = *reinterpret_cast<const float4*>(epi.bias + n0 + j * 32 + 8 * g + 4 * half);
  };
  if constexpr (EPI != EPI_QKV && EPI != EPI_RESID) load_bias();
  if constexpr (EPI == EPI_QKV && TN % 2 == 0) {
    if (epi.head_dim == 64) {
      // Heads of 64 columns: a head is n-blocks 2 jh and 2 jh + 1 of the
      // wave; this lane holds 32 of its 64 columns for token m and the lane
      // 32 away the other 32.  The paper's block adds, for K and V, the RMS
      // norm over the head (one exchange between the two lanes) and, for Q
      // and K, the rotary positions of consecutive column pairs, which stay
      // inside the lane.  Q and K rows ([head][token][64], 128 bytes each)
      // go out through a wave-private LDS slice of the idle B stages, per
      // 32-row block, and are stored as whole rows (direct stores would put
      // 32 rows' 8-byte pieces in each instruction); V's transposed stores
      // already write 64 contiguous bytes per instruction and stay direct.
      constexpr int QRB = WN * 2;                       // bytes of one staged row
      constexpr int QSLOTS = (BN * 64) / (32 * QRB);
      static_assert(QSLOTS >= 1 && (NWAVES + QSLOTS - 1) / QSLOTS <= STAGES, "QKV staging");
      const int arr = wave / QSLOTS;
      uint8_t* qbuf = (arr == 0 ? sb0 : arr == 1 ? sb1 : arr == 2 ? sb2 : sb3) +
                      (wave % QSLOTS) * (32 * QRB);
      stage_barrier();                                  // every wave is done reading the ring
      const int nq = epi.d_model, nk = epi.kv_heads * 64;
      const int ns = epi.streams > 0 ? epi.streams : 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + i * 32 + r32;
        const bool live = m < args.m;
        const int b = live && epi.rows_s ? m / epi.rows_s : 0;
        const int rr = live ? m - b * epi.rows_s : 0;         // row within the stream
        const int sf = epi.sub_n ? rr / epi.sub_n : 0;
        const int mt = rr - sf * epi.sub_n;
        const int ti = mt / epi.tok_w, tj = mt - ti * epi.tok_w;
#pragma unroll
        for (int jh = 0; jh < TN / 2; ++jh) {
          const int nh = n0 + jh * 64;                 // first column of the head
          const int which = nh < nq ? 0 : (nh < nq + nk ? 1 : 2);
          float v[2][16];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 bi = *reinterpret_cast<const float4*>(
                  epi.bias + nh + jj * 32 + 8 * g + 4 * half);
              v[jj][4 * g + 0] = acc[i][2 * jh + jj][4 * g + 0] + bi.x;
              v[jj][4 * g + 1] = acc[i][2 * jh + jj][4 * g + 1] + bi.y;
              v[jj][4 * g + 2] = acc[i][2 * jh + jj][4 * g + 2] + bi.z;
              v[jj][4 * g + 3] = acc[i][2 * jh + jj][4 * g + 3] + bi.w;
            }
          if (which != 0 && epi.kv_norm) {
            float ss = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int x = 0; x < 16; ++x) ss = fmaf(v[jj][x], v[jj][x], ss);
            ss += __shfl_xor(ss, 32);
            const float rs = rsqrtf(ss * (1.0f / 64.0f) + epi.norm_eps);
            const float* gain = which == 1 ? epi.kn_g : epi.vn_g;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const float4 gg = *reinterpret_cast<const float4*>(gain + jj * 32 + 8 * g + 4 * half);
                v[jj][4 * g + 0] *= rs * gg.x;
                v[jj][4 * g + 1] *= rs * gg.y;
                v[jj][4 * g + 2] *= rs * gg.z;
                v[jj][4 * g + 3] *= rs * gg.w;
              }
          }
          if (which != 2 && epi.rope) {
            // pair p = column / 2: temporal 0..11, token row 12..21, column 22..31
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                  // pair jj*16 + 4g + e2 (lanes 0..31) or that + 2 (lanes 32..63):
                  // both indices are compile-time, the lane picks one.
                  const int p0 = jj * 16 + 4 * g + e2;
                  const float2 c0 = rope_cs(epi, p0, ti, tj, sf);
                  const float2 c1 = rope_cs(epi, p0 + 2, ti, tj, sf);
                  const float2 cs = half ? c1 : c0;
                  const float x0 = v[jj][4 * g + 2 * e2], x1 = v[jj][4 * g + 2 * e2 + 1];
                  v[jj][4 * g + 2 * e2] = x0 * cs.x - x1 * cs.y;
                  v[jj][4 * g + 2 * e2 + 1] = x0 * cs.y + x1 * cs.x;
                }
          }
          if (which == 2) {
            if (live) {
#pragma unroll
              for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  floatx4 v4 = {v[jj][4 * g], v[jj][4 * g + 1], v[jj][4 * g + 2],
                                v[jj][4 * g + 3]};
                  qkv_store4(epi, b, rr, nh + jj * 32 + 8 * g + 4 * half, v4, write_slot);
                }
            }
          } else {
            const float sc = which == 0 ? epi.q_scale : 1.0f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                uint2 w;
                w.x = f2bf2(v[jj][4 * g] * sc, v[jj][4 * g + 1] * sc);
                w.y = f2bf2(v[jj][4 * g + 2] * sc, v[jj][4 * g + 3] * sc);
                const int c = jh * 8 + jj * 4 + g;         // 16-byte chunk of the row
                *reinterpret_cast<uint2*>(qbuf + r32 * QRB + ((c ^ (r32 & 7)) << 4) + 8 * half) = w;
              }
          }
        }
        // Read back this block's Q and K heads: lane i takes chunk i % 8 of
        // row i / 8 (+ 8 per step), so 8 lanes store one 128-byte row.
#pragma unroll
        for (int jh = 0; jh < TN / 2; ++jh) {
          const int nh = n0 + jh * 64;
          const int which = nh < nq ? 0 : (nh < nq + nk ? 1 : 2);
          if (which == 2) continue;
          const int head = which == 0 ? nh / 64 : (nh - nq) / 64;
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int row = it * 8 + (lane >> 3), c = lane & 7;
            const int cc = jh * 8 + c;
            const uint4 val = *reinterpret_cast<const uint4*>(qbuf + row * QRB + ((cc ^ (row & 7)) << 4));
            const int mrow = m0 + i * 32 + row;
            if (mrow < args.m) {
              const int sb = epi.rows_s ? mrow / epi.rows_s : 0;
              const int r2 = mrow - sb * epi.rows_s;
              uint16_t* dst =
                  which == 0
                      ? epi.out_bf16 + ((size_t)(sb * epi.heads + head) * epi.q_rows + r2) * 64
                      : epi.ring_k +
                            (((size_t)write_slot * ns + sb) * epi.kv_heads + head) * (size_t)epi.n_pad * 64 +
                            (size_t)r2 * 64;
              *reinterpret_cast<uint4*>(dst + c * 8) = val;
            }
          }
        }
      }
      return;
    }
  }
  // GELU to bf16 goes out through LDS: a lane holds 4 columns of one row,
  // so direct stores put 32 rows' 16-byte pieces in each instruction; staged
  // per 32-row block in a wave-private slice of the (now idle) B stages, a
  // row of the wave's WN columns is read back as whole 16-byte chunks and
  // stored as full 128-byte lines.  (The fp32 residual epilogue measured
  // slower this way and stays direct.)  Chunk c of staged row r sits at
  // c ^ (r & 7).
  constexpr int RB = WN * 2;                   // bytes of one staged bf16 row
  constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  constexpr int SLOTS = (BN * 64) / (32 * RB); // wave slices per B stage
  constexpr bool kStaged = EPI == EPI_GELU_BF16 && CPR >= 8 && SLOTS >= 1 &&
                           (NWAVES + (SLOTS > 0 ? SLOTS : 1) - 1) / (SLOTS > 0 ? SLOTS : 1) <= STAGES;
  if constexpr (kStaged) {
    const int arr = wave / SLOTS;
    uint8_t* buf = (arr == 0 ? sb0 : arr == 1 ? sb1 : arr == 2 ? sb2 : sb3) +
                   (wave % SLOTS) * (32 * RB);
    stage_barrier();                           // every wave is done reading the ring
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 b = bv[j][g];
          uint2 w;
          w.x = f2bf2(gelu_erf(acc[i][j][4 * g] + b.x), gelu_erf(acc[i][j][4 * g + 1] + b.y));
          w.y = f2bf2(gelu_erf(acc[i][j][4 * g + 2] + b.z), gelu_erf(acc[i][j][4 * g + 3] + b.w));
          const int c = 4 * j + g;
          *reinterpret_cast<uint2*>(buf + r32 * RB + ((c ^ (r32 & 7)) << 4) + 8 * half) = w;
        }
#pragma unroll
      for (int it = 0; it < 32 * CPR / 64; ++it) {
        const int row = (it * 64 + lane) / CPR, c = lane % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(buf + row * RB + ((c ^ (row & 7)) << 4));
        const int m = m0 + i * 32 + row;
        if (m < args.m)
          *reinterpret_cast<uint4*>(epi.out_bf16 + (size_t)m * epi.ldo + n0 + c * 8) = v;
      }
    }
    return;
  }
  if constexpr (EPI == EPI_QKV) load_bias();
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + i * 32 + r32;
      if (m < args.m) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          float4 b4[4], h4[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + j * 32 + 8 * g + 4 * half;
            b4[g] = *reinterpret_cast<const float4*>(epi.bias + n);
            h4[g] = *reinterpret_cast<const float4*>(epi.out_f32 + (size_t)m * epi.ldo + n);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            floatx4 v4 = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                          acc[i][j][4 * g + 3]};
            epi_store4<EPI>(epi, m, n0 + j * 32 + 8 * g + 4 * half, v4, write_slot, b4[g], h4[g]);
          }
        }
      }
    }
  } else {
    const float4 none = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + i * 32 + r32;
      if (m < args.m) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            floatx4 v4 = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                          acc[i][j][4 * g + 3]};
            epi_store4<EPI>(epi, m, n0 + j * 32 + 8 * g + 4 * half, v4, write_slot, bv[j][g],
                            none);
          }
      }
    }
  }
}

template <int BM, int BN, int WM_, int WN_, int ST, int MINB>
hipError_t launch_epi(int epi, const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.m + BM - 1) / BM) * (a.n / BN);
  dim3 grid(tiles), block(kWave * WM_ * WN_);
  switch (epi) {
    case EPI_F32_BIAS:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_F32_BIAS>), grid,
                         block, 0, s, a);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_RESID>), grid,
                         block, 0, s, a);
      break;
    case EPI_GELU_BF16:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_GELU_BF16>), grid,
                         block, 0, s, a);
      break;
    case EPI_QKV:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_QKV>), grid,
                         block, 0, s, a);
      break;
    case EPI_PIXELS:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_PIXELS>), grid,
                         block, 0, s, a);
      break;
    case EPI_SUBFRAMES:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM_, WN_, ST, MINB, EPI_SUBFRAMES>), grid,
                         block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Pick a tile (measured on the decode shapes at M = 8160, 3600 and 1560, for
// D = 1024 and 1536, and on the batched 480p shapes).  Eight waves per
// workgroup, two waves per SIMD, beat four waves in each of two workgroups
// per CU (1080p QKV 71.3 -> 68.2 us, XL FC2 141.5 -> 131.3 us in the
// decode).  The 128-row tiles keep every epilogue within 128 VGPRs, so that
// when a GEMM takes more than one round of tiles two workgroups share a CU
// (their LDS rings fit together) and one's epilogue overlaps the other's
// main loop (480p x 8 FC2: 153.6 us at 169 VGPRs against 132 us at 104):
//  * GELU (FC1) with >= 192 tiles of 256 x 256 rows and columns, and other
//    epilogues with >= 384 tiles of 128x256 (> 224 when n <= 1024): 128x256,
//    8 waves of 64x64, 3-stage ring (72 KB LDS).  A 256x256 FC1 tile (8 waves
//    of 128x64, 128 KB LDS) ran its own launch faster (1080p 82 against
//    91.6 us) but drew the clock down for the launches after it: the whole
//    1080p frame took 18.24 ms with it and 17.42 ms without (attention 467
//    -> 429 us, QKV 71 -> 68 us), 720p 6.55 -> 6.44 ms;
//  * >= 192 tiles of 128x128: 128x128, 8 waves of 32x64, 4-stage ring;
//  * otherwise 64x128 (4 waves of 32x64, three per CU), else 64x64.
// m_rows_alloc (rows of A) must be a multiple of the chosen BM; callers
// allocate activations in multiples of 256 rows.
hipError_t launch_gemm(int epi, const GemmArgs& a, int m_rows_alloc, hipStream_t s) {
  if (a.n <= 0 || a.k <= 0 || a.k % 32 != 0) return hipErrorInvalidValue;
  if (a.m <= 0) return hipSuccess;
  const long tiles_256 = (long)((a.m + 255) / 256) * (a.n / 256);
  const long tiles_128x256 = (long)((a.m + 127) / 128) * (a.n / 256);
  const long tiles_128 = (long)((a.m + 127) / 128) * (a.n / 128);
  const bool wide = a.n % 256 == 0 && m_rows_alloc % 128 == 0 &&
                    (epi == EPI_GELU_BF16 ? tiles_256 >= 192
                                          : tiles_128x256 >= 384 ||
                                                (a.n <= 1024 && tiles_128x256 > 224));
  if (wide) return launch_epi<128, 256, 2, 4, 3, 1>(epi, a, s);
  if (a.n % 128 == 0 && m_rows_alloc % 128 == 0 && tiles_128 >= 192)
    return launch_epi<128, 128, 4, 2, 4, 1>(epi, a, s);
  if (a.n % 128 == 0 && m_rows_alloc % 64 == 0)
    return launch_epi<64, 128, 2, 2, 4, 3>(epi, a, s);
  // 64x64 waves own 32 columns; the per-head epilogue of the paper's block
  // needs a wave to own whole 64-column heads.
  if (epi == EPI_QKV && (a.epi.kv_norm || a.epi.rope)) return hipErrorInvalidValue;
  if (a.n % 64 == 0 && m_rows_alloc % 64 == 0)
    return launch_epi<64, 64, 2, 2, 4, 2>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace fd
