// Shared device helpers and launch-parameter structs of the verify-round kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxRows = 64;
constexpr int kMaxCols = 16;
constexpr int kMaxLanes = 64;
constexpr int kBlock = 16;       // tokens per paged-KV block
constexpr int kWave = 64;
constexpr int kMaxChunk = 4096;     // largest split-KV attention chunk (positions)
constexpr int kAttnPartPad = 4;     // a chunk partial row: O[d], then m and l, then 2 pad floats
constexpr int kMaxNgram = 8;          // longest suffix the n-gram drafter looks up (SPEC_MAX_NGRAM)
constexpr int kCUs = 256;           // compute units of an MI355X (workgroup slots of one-per-CU launches)
// The round's own K/V columns are staged per lane in kStageBlocks cache-layout blocks
// aligned to absolute positions: staged block v of lane l covers positions
// 16 (kv_len / 16 + v) .. +15.  Slots before kv_len hold a copy of the committed
// prefix of that block, slots after the lane's last column hold zeros (V) or are
// unused (K); ceil((15 + kMaxCols) / 16) = 2 blocks hold any lane.
constexpr int kStageBlocks = 2;

typedef uint16_t bf16_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Packed lane-major row layout of a round, passed by value in kernel arguments.
struct RowInfo {
  int R;                         // rows
  int L;                         // lanes
  int8_t row_lane[kMaxRows];
  int8_t row_col[kMaxRows];
  int16_t lane_start[kMaxLanes + 1];
  int8_t lane_cols[kMaxLanes];
};

// ----------------------------------------------------------------------------- numerics
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN).  pk_bf16 rounds two values into one word, a in
// the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two float32 values as bf16 hi and lo words: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ float ld_act(const float* p) { return *p; }
__device__ __forceinline__ float ld_act(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ void st_act(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_act(bf16_t* p, float v) { *p = f2bf(v); }

// D = A(16x32) * B(32x16) + C with bf16 inputs and fp32 accumulation.
// Lane i supplies A row (i % 16) and B column (i % 16), eight K elements each
// (the K index of element e is 8 * (i / 16) + e for both operands); lane i
// receives D[4 * (i / 16) + e][i % 16] for e = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }

// ----------------------------------------------------------------------------- LDS DMA
// 16 bytes per lane straight into LDS (global_load_lds_dwordx4): lane t of the wave
// reads base + voff and writes bytes [16 t, 16 t + 16) of the 1 KB LDS segment at the
// wave-uniform `seg`; NT marks data streamed once (non-temporal).  The instruction's
// immediate offset would move the LDS destination too, so it is 0.  Issued as inline
// assembly so that the compiler, which cannot tell LDS ring slots apart, does not
// drain every DMA before each LDS read; completion is tracked with explicit vmcnt
// waits (wait_vm) instead.  The low 32 bits of a flat LDS address are its LDS
// offset; M0 carries it (one wait state before the load).
template <bool NT>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, char* seg) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)seg);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding, and
// for all LDS reads; the "memory" clobber keeps the compiler from moving memory
// accesses across it.  Vector memory operations complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4);   // lgkmcnt(0), expcnt unchecked
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt %0" ::"n"(imm) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that waits for this wave's LDS accesses but not for its vector
// memory loads (__syncthreads would wait for every outstanding load).
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Block-wide sum with a fixed reduction tree (deterministic); `red` holds >= 32 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ int clamp_blk(int b, int n) { return b < 0 ? 0 : (b >= n ? n - 1 : b); }

// Block-wide float64 sum with a fixed reduction tree; `red` holds >= 32 doubles.
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// (value, index) order used by every argmax: larger value wins, lower index on ties.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// ----------------------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror & Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
// Counter = (position, lane, purpose, block), key = (seed lo, seed hi).
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
constexpr uint32_t kPurposeAccept = 0u, kPurposeRace = 1u;

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = kPhiloxM0 * c[0], hi0 = __umulhi(kPhiloxM0, c[0]);
    const uint32_t lo1 = kPhiloxM1 * c[2], hi1 = __umulhi(kPhiloxM1, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += kPhiloxW0; k1 += kPhiloxW1;
  }
}

// Uniform in (0, 1), exact in float32: ((w >> 9) + 0.5) * 2^-23.
__device__ __forceinline__ float u01(uint32_t w) {
  return ((float)(w >> 9) + 0.5f) * (1.0f / 8388608.0f);
}

// ----------------------------------------------------------------------------- fragment layout
// bf16 operands of the MFMA projections live in 1 KB fragments: the 16 x 32 slab
// (16 rows x 32 consecutive k) that one operand of v_mfma_f32_16x16x32_bf16
// covers, stored lane-major, so a wave fetches an operand with one contiguous
// 1 KB load (16 B per lane).  Lane i of fragment (g, s) holds elements
// [16 g + i % 16][32 s + 8 (i / 16) + e], e = 0..7, and fragment (g, s) starts
// at element (g * KS + s) * 512 with KS = K / 32: a tile's k steps are
// contiguous, so a wave streams one contiguous region.  Weights [N][K] use it
// with g = output-feature tile (features past N zero), activations [R][K] with
// g = row tile; an activation plane holds 16 ceil(R / 16) rows.
__host__ __device__ __forceinline__ size_t frag_off(int row, int k, int KS) {
  return ((size_t)((row >> 4) * KS + (k >> 5)) * 64 + (row & 15) + 16 * ((k >> 3) & 3)) * 8 + (k & 7);
}
__host__ __device__ __forceinline__ int round16(int r) { return (r + 15) & ~15; }

// Element (r, k) of an [R][K] activation: row-major for float32 storage,
// fragment order for the bf16 planes.
__device__ __forceinline__ size_t act_index(const float*, int r, int k, int K) { return (size_t)r * K + k; }
__device__ __forceinline__ size_t act_index(const bf16_t*, int r, int k, int K) { return frag_off(r, k, K >> 5); }
// Elements per activation plane of R rows and width K.
__host__ __device__ __forceinline__ size_t act_plane(int R, int K) { return (size_t)round16(R) * K; }

// ----------------------------------------------------------------------------- activations
// A float32 activation x is handed to the MFMA projections as two bf16 planes,
// hi = bf16(x) and lo = bf16(x - hi) (x = hi + lo to 2^-17 relative).
__device__ __forceinline__ void st_planes(bf16_t* hi, size_t plane, float v) {
  const bf16_t h = f2bf(v);
  hi[0] = h;
  hi[plane] = f2bf(v - bf2f(h));
}

// Store a float32 activation: as is for an fp32 model, as hi/lo bf16 planes for a bf16 model.
__device__ __forceinline__ void st_out(float* base, size_t plane, size_t i, float v) {
  (void)plane;
  base[i] = v;
}
__device__ __forceinline__ void st_out(bf16_t* base, size_t plane, size_t i, float v) { st_planes(base + i, plane, v); }

// Four consecutive activations (r, k0 .. k0 + 3), k0 % 4 == 0, in one go: a float4
// row-major store, or one 8-byte store per bf16 plane (they share a fragment lane slot).
__device__ __forceinline__ void st_out4(float* base, size_t plane, int r, int k0, int K, const float (&v)[4]) {
  (void)plane;
  *reinterpret_cast<f32x4*>(base + (size_t)r * K + k0) = f32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void st_out4(bf16_t* base, size_t plane, int r, int k0, int K, const float (&v)[4]) {
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) split2(v[2 * i], v[2 * i + 1], hi[i], lo[i]);
  const size_t o = frag_off(r, k0, K >> 5);
  *reinterpret_cast<u32x2*>(base + o) = u32x2{hi[0], hi[1]};
  *reinterpret_cast<u32x2*>(base + plane + o) = u32x2{lo[0], lo[1]};
}

// ----------------------------------------------------------------------------- launch parameters
// Projection Y = X W^T over packed fragments.  K is a multiple of 256; split s
// of S covers 256-wide units [s U / S, (s + 1) U / S), U = K / 256.
struct ProjParams {
  const bf16_t* W0;     // packed [N][K]
  const bf16_t* W1;     // packed second matrix of a gate/up pair, or null
  const bf16_t* X;      // packed activation planes (hi, then lo)
  size_t xplane;        // elements per activation plane
  int R, N, K, S;
  int tiles;            // ceil(N / 16)
  int units;            // balanced SwiGLU launch: gate/up units (one tile of each)
  int cols;             // workgroups per split (SwiGLU and one-wave launches)
  int scols[8];         // balanced plain launch: workgroups of split s, in split order
  float* P;             // [S][R][N] float32 partial sums
  bf16_t* Y;            // SwiGLU output planes, packed with width N
  size_t yplane;
  // balanced SwiGLU launch (rem > 0): base whole units per CU, the rem units past
  // base * kCUs cut into pq K pieces; piece sums in Q [rem][pq][2][R][16], one
  // arrival counter per cut unit in cnt (zero between launches)
  int base, rem, pq;
  float* Q;
  int* cnt;
};

struct GemmF32Params {
  const float* X; const float* W0; const float* W1;
  int R, N, K;
  float* P;             // [1][R][N]
  float* Ya;            // [R][N] SwiGLU output (fp32 model)
};

// Device-side mirror of the public spec_row_stat.
struct spec_row_stat_dev {
  float max_logit;
  float lse;
  int32_t argmax;
  float z_next;
};

// Per-(row, group) partial statistics of the LM head.
struct LmPartial {
  float m;     // max logit in the group
  float se;    // sum exp((z - m) / T) over the group
  int arg;     // lowest-index argmax in the group
  float zn;    // logit of the row's next draft token if it falls in the group, else NaN
  float gk;    // best bonus race key z/T - ln(-ln U) in the group (bonus rows only)
  int gi;      // its index
  int pad0, pad1;
};

// Row statistics after reducing the LM-head partials (internal workspace form).
struct RowStat {
  float m, se, zn, gk;
  int arg, gi, pad0, pad1;
};

// Per-lane acceptance decision (internal).
struct LaneDecision {
  int committed;        // c in [1, cols]
  int resid_row;        // row whose residual must be drawn, -1 if none
  int resid_col;        // draft index i of the rejection (position kv_len + i)
  int pad;
  float m, se;          // stats of resid_row
  float pad2, pad3;
};

struct LmParams {
  const void* X;           // final hidden: packed bf16 planes (bf16 model) or [R][H] float
  size_t xplane;           // elements per plane
  int xs;                  // bf16 planes in use (1: exact bf16 hidden states, 2: hi + lo)
  const void* W;           // packed [V][H] (bf16) or row-major [V][H] float
  int R, V, H;
  int groups;              // number of partial groups per row (the grid of the sampled bf16 head)
  const int32_t* tokens;   // [R] round tokens (next-draft lookup)
  const int32_t* kv_len;   // [L]
  float inv_t;             // 1 / T (1 in greedy mode)
  int sampled;
  uint32_t key0, key1;     // Philox key
  LmPartial* part;         // [R][groups]
  RowInfo ri;
  const int32_t* counts;   // [L][V] token counts of each lane up to its anchor, or null (no penalties)
  float presence, frequency;
  // sampled bf16 head (one cooperative launch, logits kept on chip): the grid barrier's
  // counters (kCoopCounters ints, zero at launch), the reduced row statistics, the lane
  // decisions, the residual race partials [L][groups][4] and the drafter's q [R][V]
  int* bar;
  int spin_limit;          // polls per grid barrier before the error flag is raised
  RowStat* rstat;
  LaneDecision* dec;
  float* racep;
  const float* q;
};

// Counters of the sampled head's grid barriers in the workspace: group arrivals at
// barrier 1 and 2, the error flag (a barrier wait that ran out), the grid size; then, from
// int kCoopGroupBase on, the workgroup arrivals of each barrier's eight groups, each
// count in a 128-byte line of its own (barrier j, group g at kCoopGroupBase + (8 j + g) 32).
constexpr int kCoopGroups = 8;
constexpr int kCoopGroupBase = 32;
constexpr int kCoopCounters = kCoopGroupBase + 2 * kCoopGroups * 32;

// The textbook rule on one lane's rows (Leviathan et al., Def. 3.7): draft d_i is kept iff
// u * q_i(d_i) < p_{i-1}(d_i), u the Philox uniform at (seed; position kv_len + i, lane,
// accept), p = softmax(z / T) from the row statistics.  qd(r) is the drafter's q of row r
// at its own draft token (0 for a token outside the vocabulary).  Returns the decision;
// with o non-null the kept drafts and, when every draft is kept, the bonus token (the
// race winner of the lane's last row) go to o.  rs may point to global memory or LDS.
template <typename QD>
__device__ __forceinline__ LaneDecision decide_sampled(const RowStat* rs, const int32_t* tokens, const int32_t* kv_len,
                                                       QD qd, float inv_t, uint32_t key0, uint32_t key1,
                                                       const RowInfo& ri, int l, int32_t* o) {
  const int r0 = ri.lane_start[l], k = ri.lane_cols[l] - 1;
  LaneDecision d;
  d.resid_row = -1; d.resid_col = 0; d.pad = 0; d.m = 0.f; d.se = 1.f; d.pad2 = d.pad3 = 0.f;
  const uint32_t kvl = (uint32_t)kv_len[l];
  int i = 1;
  for (; i <= k; ++i) {
    const RowStat s = rs[r0 + i - 1];
    const int di = tokens[r0 + i];
    uint32_t c[4] = {kvl + (uint32_t)i, (uint32_t)l, kPurposeAccept, 0u};
    philox4x32_10(c, key0, key1);
    const float u = u01(c[0]);
    const float pd = isnan(s.zn) ? 0.f : expf((s.zn - s.m) * inv_t) / s.se;
    if (u * qd(r0 + i) < pd) {
      if (o) o[i - 1] = di;
      continue;
    }
    d.resid_row = r0 + i - 1;
    d.resid_col = i;
    d.m = s.m;
    d.se = s.se;
    break;
  }
  if (i > k) {
    if (o) o[k] = rs[r0 + k].gi;   // bonus token from p_k
    d.committed = k + 1;
  } else {
    d.committed = i;               // token i - 1 is the residual draw
  }
  return d;
}
// Residual race of an fp32 model (recomputes the rejected row's logits).
struct RaceParams {
  const void* X;           // the round's hidden rows [R][H] float
  const void* W;           // row-major [V][H] float
  int R, V, H, L;
  int groups;
  const float* q;          // [R][V]
  const int32_t* kv_len;
  float inv_t;
  uint32_t key0, key1;
  const LaneDecision* dec; // [L]
  float* part;             // [L][groups][4]: residual key, index, fallback key, index
  RowInfo ri;
  const int32_t* tokens;   // [R] round tokens (the drafts before the rejected row)
  const int32_t* counts;   // [L][V] or null, as LmParams
  float presence, frequency;
};

// Presence / frequency penalty of one row: row j of a lane conditions on the lane's
// tokens up to its anchor (cnt) and on the round's drafts d_1 .. d_j (lane_tokens[1 .. j]),
// so a token seen c times there loses presence * [c > 0] + frequency * c.
struct RowPenalty {
  const int32_t* cnt;           // the lane's counts row, null: no penalty
  const int32_t* lane_tokens;   // the lane's round tokens (anchor first)
  int j;
  float presence, frequency;
};

__device__ __forceinline__ RowPenalty row_penalty(const int32_t* counts, int V, const int32_t* tokens,
                                                  const RowInfo& ri, int r, float presence, float frequency) {
  RowPenalty rp;
  const int l = ri.row_lane[r];
  rp.cnt = counts ? counts + (size_t)l * V : nullptr;
  rp.lane_tokens = tokens + ri.lane_start[l];
  rp.j = ri.row_col[r];
  rp.presence = presence;
  rp.frequency = frequency;
  return rp;
}

__device__ __forceinline__ float penalty_of(int c, const RowPenalty& rp) {
  return (c > 0 ? rp.presence : 0.f) + rp.frequency * (float)c;
}

__device__ __forceinline__ float penalized(float z, int v, const RowPenalty& rp) {
  int c = rp.cnt[v];
  for (int i = 1; i <= rp.j; ++i) c += rp.lane_tokens[i] == v;
  return z - penalty_of(c, rp);
}

// Penalties of the tokens v0[t] .. v0[t] + 3 of T groups of four (each v0 a multiple of
// 4 and at most V - 4; a lane's count row is 16-byte aligned): one 16-byte count load per
// group and one pass over the row's drafts, whose loads do not depend on each other.
template <int T>
__device__ __forceinline__ void penalties4(const RowPenalty& rp, const int (&v0)[T], float (&pz)[T][4]) {
  int c[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int4 cv = *reinterpret_cast<const int4*>(rp.cnt + v0[t]);
    c[t][0] = cv.x; c[t][1] = cv.y; c[t][2] = cv.z; c[t][3] = cv.w;
  }
#pragma unroll
  for (int i = 1; i < kMaxCols; ++i) {
    const int d = rp.lane_tokens[min(i, rp.j)];   // index within the lane's columns
    const bool on = i <= rp.j;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) c[t][e] += (on && d == v0[t] + e) ? 1 : 0;
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) pz[t][e] = penalty_of(c[t][e], rp);
}

// Where the QKV epilogue stages a round's own K/V columns from: the lanes' cache
// lengths and the committed prefix of each lane's first staged block (layer slices).
struct KvStage {
  const int32_t* kv_len;
  const int32_t* block_table;   // [L][max_blocks]
  int max_blocks, n_blocks;
  const void* kpool;            // [n_blocks][nkv][16][d]
  const void* vpool;            // [n_blocks][nkv][d][16]
};

// Float index of (query row m, column f) in a chunk partial slot: four-float granules,
// granule-major over the slot's 64 rows, so a wave's 16-byte stores of 16 consecutive
// rows are 256 contiguous bytes.  Columns d .. d + 1 hold the row's max and sum.
__host__ __device__ __forceinline__ size_t part_index(int m, int f) {
  return ((size_t)(f >> 2) * 64 + m) * 4 + (f & 3);
}

struct AttnParams {
  const float* q;         // [R][nq][d] float32 queries
  const void* sk;         // staged K [L][kStageBlocks][nkv][16][d] (cache block layout)
  const void* sv;         // staged V [L][kStageBlocks][nkv][d][16]
  const void* kpool;      // layer slice [n_blocks][nkv][16][d]
  const void* vpool;      // layer slice [n_blocks][nkv][d][16]
  const int32_t* block_table;
  int max_blocks, n_blocks;
  const int32_t* kv_len;
  int nq, nkv, G, d;
  int chunk;              // positions per workgroup chunk
  int n_chunks;           // chunks per lane (partial slots)
  float scale_log2;       // log2(e) / sqrt(d)
  float* part;            // [L][nkv][n_chunks] slots of 64 rows x (d + kAttnPartPad) floats, part_index order
  RowInfo ri;
  // bf16 model: the attention kernel forms the queries and the staged columns itself from
  // the QKV projection's split partials (null: q, sk and sv are already written)
  const float* P;         // [S][R][(nq + 2 nkv) d]
  int S;
  const double* rope;     // [R][d / 2] (cos, sin) in float64, or null (no positional encoding)
  int window;             // 0: full attention; W > 0: a row at position P sees P - W + 1 .. P
};

}  // namespace sv
