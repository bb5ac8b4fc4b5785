// Verify attention (gfx950).
//
// "Speculative decoding" (gpillon.github.io/ignis), "One round, step by step",
// step 3: all of a lane's columns (anchor plus drafts) go through the layer in
// one pass; column j attends to the lane's committed cache and to its own
// columns 0..j (causal among the columns of the round).
//
// Split-KV: the positions of a lane are cut into chunks of `chunk` absolute
// positions, each chunk yields a partial (O, max, sum) per query row, and the
// combine kernel merges the partials in chunk order.  All (k+1) x G query rows
// of a lane/kv-head pair are processed together, so every K/V byte of the lane
// is read once per layer.  The round's own columns are staged in cache-layout
// blocks aligned to absolute positions, so a 16-position block is either a
// committed block of the paged cache or a staged block, and which positions an
// online softmax visits, in which order, is fixed by absolute position.  A row's
// result is therefore independent of how many columns the round carries and of
// whether a key is still staged or already committed.
//
// bf16 path (head_dim 128): two waves per query tile (16 of the lane's (k+1) x G
// query rows), one per 32-position half of every 64-position stage, each with an
// online softmax of its own that is merged with the other's at the chunk end.  Per
// 32 positions:
//   S^T[pos][query] = K . Q^T with v_mfma_f32_16x16x32_bf16 (K rows = A; the
//   float32 queries = B, as bf16 hi + lo planes);
//   P = exp2(S * log2(e)/sqrt(d) - m) in fp32, split into bf16 hi + lo;
//   O^T[d][query] += V^T . P^T.  The V pool is stored d-major inside a block
//   ([d][16 slots]) so that V^T rows are contiguous.
// fp32 path: one workgroup per chunk, its four waves take consecutive quarters.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace sv {

constexpr int kAttnStages = 4;       // LDS ring depth (64-position stages) of the bf16 kernel
constexpr int kAttnWgBlocks = 2048;  // most cache blocks one workgroup's chunk range may span

// Values of lanes i and i ^ 16 (x16), i and i ^ 32 (x32), as (lower lane, upper lane).
__device__ __forceinline__ void pair16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// max / sum over the four lanes kq = 0..3 of a query column (lanes r, r + 16, r + 32, r + 48)
__device__ __forceinline__ float col_max(float v) {
  float a, b;
  pair16(v, a, b);
  v = fmaxf(a, b);
  pair32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float col_sum(float v) {
  float a, b;
  pair16(v, a, b);
  v = a + b;
  pair32(v, a, b);
  return a + b;
}

// ---------------------------------------------------------------- QKV post-processing
// A bf16 model's attention kernel takes the QKV projection's split partials directly:
// each value is the sum of the S partials in split order in float64, rounded once to
// float; q and k are then rotated (rotate-half RoPE: the token positions are among the
// per-token inputs of the FreeToken issue's "Flow") in float64 and rounded to float, k and
// v to bf16 for the cache.

typedef double f64x2 __attribute__((ext_vector_type(2)));

// Four consecutive floats summed over the splits s = 0 .. S - 1 in split order in float64,
// rounded once: the first OB splits come loaded (v[b] = split min(b, S - 1)), later ones
// (none while the split rule caps the QKV projection at four) are read here from src + s ss.  Selects rather than branches, so that the compiler keeps
// the loads of v where the caller issued them.
template <int OB>
__device__ __forceinline__ f32x4 split_sum(const f32x4 (&v)[OB], const float* src, size_t ss, int S) {
  double a[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = (double)v[0][e];
#pragma unroll
  for (int b = 1; b < OB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = b < S ? a[e] + (double)v[b][e] : a[e];
  for (int b = OB; b < S; ++b) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(src + (size_t)b * ss);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += (double)w[e];
  }
  return f32x4{(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
}

// Two bf16 values in one word, a at the lower address.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// (a, b) = elements i and i + d/2 of one head: rotated by the angle of (cos c, sin sn).
__device__ __forceinline__ void rotate_half(float& a, float& b, double c, double sn) {
  const double av = (double)a, bv = (double)b;
  a = (float)(av * c - bv * sn);
  b = (float)(bv * c + av * sn);
}

// rotate_half by the loaded angle cs = (cos, sin) when `on`, else (a, b) unchanged (a
// select: cs holds no angle then).
__device__ __forceinline__ void rotate_half_if(bool on, float& a, float& b, f64x2 cs) {
  float x = a, y = b;
  rotate_half(x, y, cs[0], cs[1]);
  a = on ? x : a;
  b = on ? y : b;
}

// bf16 verify attention, one workgroup per (chunk range, kv head, lane).  The
// workgroup streams its range of chunks as 64-position stages through a
// kAttnStages-deep LDS ring filled by DMA (three stages in flight while one is
// consumed) and writes a partial at every chunk end, so a row's result depends
// only on the fixed chunk grid.
//
// Work split: eight waves, two per query tile q (rows 16 q .. 16 q + 15 of the
// lane's (k+1) x G query rows): half h = 0, 1 of the tile takes positions
// 32 h .. 32 h + 31 of every stage with an online softmax of its own, so no wave
// needs anything from another within a stage and P never leaves registers.  The two
// halves are merged exactly at the chunk end.  Half 0 of tile q runs on wave q and
// half 1 on wave 4 + (q + 2) % 4, so one or two tiles occupy distinct SIMDs.  Waves
// past the lane's query tiles only copy.
//
// The S^T tiles are arranged so that their MFMA output is the B operand of the PV
// product as is: for half h, tile X takes A-operand row r from position
// 32 h + 8 (r / 4) + r % 4 and tile Y from the same plus 4, so lane i receives
// positions 32 h + 8 (i / 16) + e (X) and + 4 + e (Y), e = 0..3 -- exactly the K
// indices 8 (i / 16) .. + 7 it supplies to the PV MFMA, in position order.
//
// LDS stage: K [64 positions][256 B] with 16-byte chunk c of position p stored at
// chunk c ^ f(p), f(p) = (p & 3) | ((p >> 3) & 3) << 2, which is r for the row r of
// every S^T tile, so the A-operand reads are free of bank conflicts; V^T block-major
// [4 blocks][128 d][32 B] with the two 16-byte halves of row d swapped when d & 4.
// Wave w < 4 DMAs the K rows of block w of each stage, wave 4 + b the V^T rows of
// block b; one workgroup barrier per stage publishes the stage and frees the slot the
// previous stage used.  Every DMA reads 1 KB from one cache block: a wave-uniform
// block address plus per-lane offsets fixed for the whole kernel.
__global__ __launch_bounds__(512) void k_attn_bf16(AttnParams p) {
  constexpr int D = 128, STEP = 64, NS = kAttnStages, PW = kAttnPartPad + D;
  constexpr int KBYTES = STEP * D * 2, SBYTES = 2 * KBYTES;
  constexpr int NST = 9;    // store instructions of one chunk partial (half-0 waves)
  __shared__ __attribute__((aligned(1024))) char ring[NS * SBYTES];
  __shared__ int sblk[kAttnWgBlocks];                                 // committed block ids of the range
  __shared__ float2 mlx[4][16];                                       // half 1's (max, sum) at chunk ends
  const int x = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int nch = (end + p.chunk - 1) / p.chunk;
  // sliding window: no row of the lane sees a position below lo, so the chunks below cl
  // are skipped and the lane's first range starts at the stage holding lo
  const int lo = p.window > 0 ? max(0, kvl - p.window + 1) : 0;
  const int cl = lo / p.chunk, nw = nch - cl;
  const int c0 = cl + x * nw / (int)gridDim.x, c1 = cl + (x + 1) * nw / (int)gridDim.x;
  if (c0 >= c1) return;
  const int first = max(c0 * p.chunk, lo / STEP * STEP);                // first position of the range
  const int tb = (first - c0 * p.chunk) / STEP;                         // stages of chunk c0 skipped
  const int T = (min(c1 * p.chunk, end) - first + STEP - 1) / STEP;     // stages of the range
  const int cs = p.chunk / STEP;                                        // stages per chunk
  const int fb = first >> 4, b0 = kvl >> 4;   // blocks >= b0 come from the staged columns
  const int* bt = p.block_table + (size_t)l * p.max_blocks;
  const int nkv = p.nkv, Mq = cols * p.G;
  const int h = wave >> 2;                    // half of the stage's positions
  const int qtile = h ? ((wave + 2) & 3) : wave;
  const bool active = 16 * qtile < Mq;        // the wave has query rows (wave-uniform)
  const float scale = p.scale_log2;
  const char* Kp = reinterpret_cast<const char*>(p.kpool);
  const char* Vp = reinterpret_cast<const char*>(p.vpool);
  constexpr int BLOCK_BYTES = kBlock * D * 2;
  // Blocks below b0 are committed cache blocks.  Block b0 and every block after it are
  // fetched from the lane's boundary cache block (its committed prefix, slots below
  // kv_len % 16, is exact); the round's own columns are then written into the LDS stage
  // over it, and V is zeroed at positions past the lane's end (K there is masked).
  const int blk0 = clamp_blk(bt[min(b0, p.max_blocks - 1)], p.n_blocks);
  // per-lane DMA offsets, fixed for the kernel.  K waves: segment i holds positions
  // 4 i .. 4 i + 3 of block w (stage position p = 16 w + 4 i + lane / 16; LDS chunk
  // lane % 16 receives chunk (lane % 16) ^ f(p)).  V waves: segment i holds rows
  // 32 i .. 32 i + 31 of block w - 4 (lane t: row t / 2, LDS half t & 1 receives half
  // (t & 1) ^ (row / 4 & 1)).
  const int bw = wave & 3;                    // the block this wave copies
  const char* pool = h ? Vp : Kp;             // its pool
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * i + (lane >> 4), ps = 16 * bw + q;
    const int f = (ps & 3) | (((ps >> 3) & 3) << 2);
    off[i] = h ? 1024 * i + (lane >> 1) * 32 + ((((lane & 1) ^ ((lane >> 3) & 1))) << 4)
               : q * 256 + (((lane & 15) ^ f) << 4);
  }
  // ---- DMA of this wave's part of stage t into ring slot t % NS, 4 instructions
  auto issue = [&](int t) {
    char* dst = ring + (t % NS) * SBYTES + h * KBYTES + 4096 * bw;
    const int b = fb + 4 * t + bw;
    const int id = __builtin_amdgcn_readfirstlane(b < b0 ? sblk[b - fb] : blk0);
    const char* src = pool + ((size_t)id * nkv + g) * BLOCK_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16<true>(src, off[i], dst + 1024 * i);
  };

  // ---- prologue, one round trip before the first DMA (the compiler's waits for these
  // loads do not count the DMAs, so every load is consumed before the first DMA): the
  // block ids of the range; for workgroups whose range reaches position kv_len, the
  // round's own columns; the wave's queries
  constexpr int IPT = kAttnWgBlocks / 512;
  const int ncommit = min(4 * T, b0 - fb);
  int idv[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int i = min(tid + 512 * k, max(ncommit - 1, 0));   // fb + i < max_blocks
    idv[k] = bt[fb + i];
  }
  const int N = (p.nq + 2 * nkv) * D;
  const size_t ss = (size_t)p.ri.R * N;
  // Every load of the prologue is issued before the first use of any: the split partials
  // of up to OB splits and the RoPE angles of the own columns and of the queries.  The
  // sums take the loaded splits through selects, not branches, so that no load is sunk to
  // its use (a chain of memory round trips otherwise).
  constexpr int OB = 4;                        // splits requested up front
  const bool rope = p.rope != nullptr;
  // without RoPE the angle loads read this (valid) row instead and are discarded
  const f64x2* rdummy = reinterpret_cast<const f64x2*>(p.P + (size_t)rs * N);
  auto rope_at = [&](int row, int i0) -> const f64x2* {
    return rope ? reinterpret_cast<const f64x2*>(p.rope + ((size_t)row * (D / 2) + i0) * 2) : rdummy;
  };
  // own columns: item k of this thread (k = 0, 1) is (column j, rotation pairs i0 .. i0 + 3
  // of K) for items below cols 16, then (column j, elements i0 .. i0 + 3 of V)
  const bool own = min(c1 * p.chunk, end) > kvl;
  const int nownk = cols * 16, nown = cols * 48;
  f32x4 ownraw[2][2][OB];
  f64x2 ownrt[2][4];
  auto own_item = [&](int it, bool& isk, int& j, int& i0) {
    isk = it < nownk;
    const int jt = isk ? it : it - nownk, per = isk ? 16 : 32;
    j = jt / per;
    i0 = 4 * (jt - j * per);
  };
  auto own_src = [&](int it, int half) -> const float* {
    bool isk;
    int j, i0;
    own_item(it, isk, j, i0);
    const float* row = p.P + (size_t)(rs + j) * N;
    return isk ? row + (size_t)(p.nq + g) * D + i0 + half * (D / 2) : row + (size_t)(p.nq + nkv + g) * D + i0;
  };
  if (own) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && nown <= 512) break;        // one item per thread
      const int it = min(tid + 512 * k, nown - 1);
      bool isk;
      int j, i0;
      own_item(it, isk, j, i0);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int b = 0; b < OB; ++b)   // V items read their elements twice (the second copy is unused)
          ownraw[k][hf][b] = *reinterpret_cast<const f32x4*>(own_src(it, isk ? hf : 0) + (size_t)min(b, p.S - 1) * ss);
      const f64x2* rt = isk ? rope_at(rs + j, i0) : rdummy;
#pragma unroll
      for (int e = 0; e < 4; ++e) ownrt[k][e] = rt[e];
    }
  }
  // queries, each element once per workgroup: item it (two per thread) = (query row mr,
  // rotation pairs i0 .. i0 + 3)
  f32x4 qraw2[2][2][OB];
  f64x2 qrt[2][4];
  const float* qrow[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int it = min(tid + 512 * k, Mq * 16 - 1);
    const int mr = it >> 4, i0 = 4 * (it & 15);
    const int jr = mr / p.G, hr = mr - jr * p.G;
    qrow[k] = p.P + (size_t)(rs + jr) * N + (size_t)(g * p.G + hr) * D + i0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int b = 0; b < OB; ++b)
        qraw2[k][hf][b] = *reinterpret_cast<const f32x4*>(qrow[k] + hf * (D / 2) + (size_t)min(b, p.S - 1) * ss);
    const f64x2* rt = rope_at(rs + jr, i0);
#pragma unroll
    for (int e = 0; e < 4; ++e) qrt[k][e] = rt[e];
  }
  // the float32 queries go to ring slot NS - 1 (untouched until the loop's first
  // barrier), float4 group c of row mr at c ^ (mr & 31)
  float* qs = reinterpret_cast<float*>(ring + (NS - 1) * SBYTES);   // [64][128] floats
  float qv[2][2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 v = split_sum<OB>(qraw2[k][hf], qrow[k] + hf * (D / 2), ss, p.S);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[k][hf][e] = v[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) rotate_half_if(rope, qv[k][0][e], qv[k][1][e], qrt[k][e]);
  }
  // own columns: sums in split order in float64, rotation, bf16; held in registers until
  // the column's stage is in LDS
  u32x4 ownv[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  if (own) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && nown <= 512) break;
      const int it = min(tid + 512 * k, nown - 1);
      bool isk;
      int j, i0;
      own_item(it, isk, j, i0);
      float v[2][4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 w = split_sum<OB>(ownraw[k][hf], own_src(it, isk ? hf : 0), ss, p.S);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[hf][e] = w[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) rotate_half_if(isk && rope, v[0][e], v[1][e], ownrt[k][e]);
      ownv[k] = isk ? u32x4{pack_bf16(v[0][0], v[0][1]), pack_bf16(v[0][2], v[0][3]), pack_bf16(v[1][0], v[1][1]),
                            pack_bf16(v[1][2], v[1][3])}
                    : u32x4{pack_bf16(v[0][0], v[0][1]), pack_bf16(v[0][2], v[0][3]), 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int it = tid + 512 * k;
    if (it < Mq * 16) {
      const int mr = it >> 4, c = it & 15;   // float4 groups c (pairs 4c ..) and c + 16 (their partners)
      *reinterpret_cast<f32x4*>(qs + mr * D + 4 * (c ^ (mr & 31))) =
          f32x4{qv[k][0][0], qv[k][0][1], qv[k][0][2], qv[k][0][3]};
      *reinterpret_cast<f32x4*>(qs + mr * D + 4 * ((c + 16) ^ (mr & 31))) =
          f32x4{qv[k][1][0], qv[k][1][1], qv[k][1][2], qv[k][1][3]};
    }
  }
#pragma unroll
  for (int k = 0; k < IPT; ++k)
    if (tid + 512 * k < ncommit) sblk[tid + 512 * k] = clamp_blk(idv[k], p.n_blocks);
  if (own) {
#pragma unroll
    for (int k = 0; k < 2; ++k) asm volatile("" ::"v"(ownv[k]));
  }
  wg_barrier();   // block ids and queries staged
  for (int t = 0; t < NS - 1 && t < T; ++t) issue(t);
  // the wave's queries: elements kq 8 + 32 ds + e of row m (float4 groups 2 kq + 8 ds and
  // + 1), read back before the loop's first barrier frees slot NS - 1 for the DMAs
  const int m = 16 * qtile + r16;              // the lane's query row
  f32x4 qraw[8];
  {
    const int mc = min(m, Mq - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 2 * kq + 8 * (i >> 1) + (i & 1);
      qraw[i] = *reinterpret_cast<const f32x4*>(qs + mc * D + 4 * (c ^ (mc & 31)));
    }
  }
  const bool valid = m < Mq;
  const int lim = valid ? kvl + m / p.G : -1;  // last position the row attends to
  u32x4 qh[4], ql[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    const f32x4 a = qraw[2 * ds], b = qraw[2 * ds + 1];
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hw, lw;
      split2(v[2 * i], v[2 * i + 1], hw, lw);
      qh[ds][i] = valid ? hw : 0u;
      ql[ds][i] = valid ? lw : 0u;
    }
  }

  // Writes the own columns of stage t (positions s0 .. s0 + 63) into its ring slot and
  // zeroes V past the lane's end; the caller's barrier publishes them.
  auto patch = [&](int t) {
    const int s0 = first + STEP * t;
    char* sK = ring + (t % NS) * SBYTES;
    char* sV = sK + KBYTES;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int it = tid + 512 * k;
      if (it >= nown) continue;
      const bool isk = it < nownk;
      const int jt = isk ? it : it - nownk, per = isk ? 16 : 32;
      const int j = jt / per, i0 = 4 * (jt - j * per);
      const int ps = kvl + j - s0;
      if (ps < 0 || ps >= STEP) continue;
      if (isk) {
        const int f = (ps & 3) | (((ps >> 3) & 3) << 2), c = i0 >> 3, o = (i0 & 7) * 2;
        *reinterpret_cast<u32x2*>(sK + ps * 256 + ((c ^ f) << 4) + o) = u32x2{ownv[k][0], ownv[k][1]};
        *reinterpret_cast<u32x2*>(sK + ps * 256 + (((8 + c) ^ f) << 4) + o) = u32x2{ownv[k][2], ownv[k][3]};
      } else {
        const int bb = ps >> 4, sl = ps & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = i0 + e;
          const uint32_t w = ownv[k][e >> 1];
          *reinterpret_cast<bf16_t*>(sV + bb * 4096 + d * 32 + (((sl >> 3) ^ ((d >> 2) & 1)) << 4) + (sl & 7) * 2) =
              (bf16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
        }
      }
    }
    // V rows past the end: thread = (block bb of the stage, row d)
    {
      const int bb = tid >> 7, d = tid & 127;
      const int sz = min(max(end - (s0 + 16 * bb), 0), 16);   // first slot to zero
      char* vrow = sV + bb * 4096 + d * 32;
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        char* half = vrow + ((hs ^ ((d >> 2) & 1)) << 4);
        if (8 * hs >= sz) {
          *reinterpret_cast<u32x4*>(half) = u32x4{0u, 0u, 0u, 0u};
        } else if (8 * hs + 8 > sz) {
          for (int e = sz - 8 * hs; e < 8; ++e) *reinterpret_cast<bf16_t*>(half + 2 * e) = (bf16_t)0;
        }
      }
    }
  };

  // running max (raw score units), this lane's part of the row sum, O^T[16 dt + 4 kq + e][m]
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int t) {
    const char* sK = ring + (t % NS) * SBYTES;
    const char* sV = sK + KBYTES;
    // S^T tiles X (y = 0) and Y (y = 1) of the half: lane i reads row r16 = position
    // 32 h + 8 (r16 / 4) + r16 % 4 + 4 y, whose chunks are swizzled by f = r16
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const char* kr = sK + (32 * h + 8 * (r16 >> 2) + (r16 & 3)) * 256;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 kf[2];
#pragma unroll
      for (int y = 0; y < 2; ++y) kf[y] = *reinterpret_cast<const u32x4*>(kr + 4 * y * 256 + (((4 * ds + kq) ^ r16) << 4));
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        sc[y] = mfma_bf16(kf[y], ql[ds], sc[y]);
        sc[y] = mfma_bf16(kf[y], qh[ds], sc[y]);
      }
    }
    // lane value e of tile y is position 32 h + 8 kq + 4 y + e; positions past a query's
    // own column are masked, and a stage below kv_len needs none
    const int p0 = first + STEP * t + 32 * h + 8 * kq;
    if (first + STEP * t + STEP > kvl) {
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[y][e] = p0 + 4 * y + e <= lim ? sc[y][e] : -INFINITY;
    }
    // positions below a query's window (W positions ending at its own column); the
    // highest window start of the lane is end - W
    if (p.window > 0 && first + STEP * t < end - p.window) {
      const int lw = lim - p.window + 1;
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[y][e] = p0 + 4 * y + e >= lw ? sc[y][e] : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    const float mnew = fmaxf(mrun, col_max(mx));
    float pr[2][4];
    float alpha = 1.f;
    if (mnew == -INFINITY) {
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[y][e] = 0.f;
    } else {
      // exp2(scale (s - m)) with the raw v_exp_f32: the arguments are at most a rounding
      // of m * scale above zero, results below 2^-126 flush to 0
      const float ms = mnew * scale;
      alpha = __builtin_amdgcn_exp2f(fmaf(mrun, scale, -ms));
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[y][e] = __builtin_amdgcn_exp2f(fmaf(sc[y][e], scale, -ms));
    }
    lrun = lrun * alpha + (((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3])));
    mrun = mnew;
    // P^T as bf16 hi + lo B operands: K index 8 kq + e from X, 8 kq + 4 + e from Y
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(pr[i >> 1][2 * (i & 1)], pr[i >> 1][2 * (i & 1) + 1], hw[i], lw[i]);
    const u32x4 ph = u32x4{hw[0], hw[1], hw[2], hw[3]}, pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
    // O *= alpha, skipped when no row of the wave has a new maximum (alpha is then 1)
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
    }
    // O^T[d][m] += V^T[d][keys] P^T[keys][m]: lane i supplies row d = 16 dt + r16 of V^T at
    // positions 32 h + 8 kq .. +7 (half kq & 1 of block 2 h + kq / 2)
    const char* vr = sV + 4096 * (2 * h + (kq >> 1)) + r16 * 32 + (((kq & 1) ^ ((r16 >> 2) & 1)) << 4);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4 vf = *reinterpret_cast<const u32x4*>(vr + 16 * dt * 32);
      O[dt] = mfma_bf16(vf, pl, O[dt]);
      O[dt] = mfma_bf16(vf, ph, O[dt]);
    }
  };

  int t_store = -NS;     // iteration of this wave's last chunk-partial stores
  const bool stores = active && h == 0;
  for (int t = 0; t < T; ++t) {
    // this wave's DMAs of stage t are complete once at most (stages issued after it)
    // x 4 DMAs, plus chunk-partial stores issued after it, are outstanding
    const int after = min(T, t + NS - 1) - (t + 1);
    if (t - t_store <= NS - 1) {
      if (after >= 2) wait_vm<8 + NST>();
      else if (after == 1) wait_vm<4 + NST>();
      else wait_vm<NST>();
    } else {
      if (after >= 2) wait_vm<8>();
      else if (after == 1) wait_vm<4>();
      else wait_vm<0>();
    }
    wg_barrier();                            // stage t is in LDS; stage t - 1 is consumed
    if (t + NS - 1 < T) issue(t + NS - 1);   // into the slot stage t - 1 used
    if (own && first + STEP * t + STEP > kvl) {
      patch(t);
      wg_barrier();                          // the own columns are in the stage
    }
    if (active) compute(t);
    if ((tb + t) % cs == cs - 1 || t == T - 1) {
      // chunk end: half 1 hands its (O, max, sum) to half 0 through the slot of stage t
      // (free once every wave is past this barrier; the next issue into it follows the
      // next stage's barrier), half 0 merges and writes the tile's partial
      wg_barrier();
      float* xo = reinterpret_cast<float*>(ring + (t % NS) * SBYTES) + qtile * 2048;
      const float lt = col_sum(lrun);
      if (active && h == 1) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(xo + (dt * 64 + lane) * 4) = O[dt];
        if (kq == 0) mlx[qtile][r16] = float2{mrun, lt};
      }
      wg_barrier();
      if (stores) {
        const float2 o1 = mlx[qtile][r16];
        const float M = fmaxf(mrun, o1.x);
        float f0 = 0.f, f1 = 0.f;
        if (M != -INFINITY) {
          const float ms = M * scale;
          f0 = __builtin_amdgcn_exp2f(fmaf(mrun, scale, -ms));
          f1 = __builtin_amdgcn_exp2f(fmaf(o1.x, scale, -ms));
        }
        const int c = c0 + (tb + t) / cs;
        float* slot = p.part + (((size_t)l * nkv + g) * p.n_chunks + c) * 64 * PW;
        // rows past the lane's queries are skipped; row 16 q is always written (never
        // read when invalid) so that every store instruction has an active lane
        if (valid || r16 == 0) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(xo + (dt * 64 + lane) * 4);
            *reinterpret_cast<f32x4*>(slot + part_index(m, 16 * dt + 4 * kq)) = O[dt] * f0 + b1 * f1;
          }
          *reinterpret_cast<f32x4*>(slot + part_index(m, D)) = f32x4{M * scale, lt * f0 + o1.y * f1, 0.f, 0.f};
        }
        t_store = t;
      }
      mrun = -INFINITY;
      lrun = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // the own columns' K and V for the commit: staged block (kv_len % 16 + j) / 16, slot
  // (kv_len % 16 + j) % 16, in the cache's block layout
  if (own) {
    bf16_t* SKg = reinterpret_cast<bf16_t*>(const_cast<void*>(p.sk));
    bf16_t* SVg = reinterpret_cast<bf16_t*>(const_cast<void*>(p.sv));
    const int pre = kvl & 15;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int it = tid + 512 * k;
      if (it >= nown) continue;
      const bool isk = it < nownk;
      const int jt = isk ? it : it - nownk, per = isk ? 16 : 32;
      const int j = jt / per, i0 = 4 * (jt - j * per);
      const int slot = pre + j, sl = slot & 15;
      const size_t sb = (size_t)kStageBlocks * l + (slot >> 4);
      if (isk) {
        bf16_t* dst = SKg + ((sb * nkv + g) * kBlock + sl) * D + i0;
        *reinterpret_cast<u32x2*>(dst) = u32x2{ownv[k][0], ownv[k][1]};
        *reinterpret_cast<u32x2*>(dst + D / 2) = u32x2{ownv[k][2], ownv[k][3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = ownv[k][e >> 1];
          SVg[((sb * nkv + g) * D + i0 + e) * kBlock + sl] = (bf16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
        }
      }
    }
  }
}

// fp32 model: VALU, one query row at a time per wave, 64 positions per step (lane = position).
__global__ __launch_bounds__(256) void k_attn_f32(AttnParams p) {
  extern __shared__ float lds[];   // [4][Mq][d + 2]
  const int c = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int D = p.d, PW = D + kAttnPartPad;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int pos0 = c * p.chunk;
  if (pos0 >= end) return;
  const int lo = p.window > 0 ? max(0, kvl - p.window + 1) : 0;   // no row sees a position below lo
  if (pos0 + p.chunk <= lo) return;
  const int Mq = cols * p.G;
  const int wlen = p.chunk >> 2;
  const int wb = pos0 + wave * wlen, we = min(wb + wlen, end);
  const int* bt = p.block_table + (size_t)l * p.max_blocks;
  const float* Qp = reinterpret_cast<const float*>(p.q);
  const float* Kp = reinterpret_cast<const float*>(p.kpool);
  const float* Vp = reinterpret_cast<const float*>(p.vpool);
  const float* SK = reinterpret_cast<const float*>(p.sk);
  const float* SV = reinterpret_cast<const float*>(p.sv);
  const int nkv = p.nkv;
  for (int m = 0; m < Mq; ++m) {
    const int j = m / p.G, hh = m - j * p.G;
    const float* q = Qp + ((size_t)(rs + j) * p.nq + g * p.G + hh) * D;
    const int lim = kvl + j;
    const int lw = p.window > 0 ? lim - p.window + 1 : 0;   // the row's window starts at lw
    float mr = -INFINITY;
    double lr = 0.0, o0 = 0.0, o1 = 0.0;
    for (int p0 = wb; p0 < we; p0 += 64) {
      const int pos = p0 + lane;
      const bool valid = pos < we && pos <= lim && pos >= lw;
      float s = -INFINITY;
      if (valid) {
        const float* kr;
        if (pos < kvl) kr = Kp + (((size_t)clamp_blk(bt[pos >> 4], p.n_blocks) * nkv + g) * kBlock + (pos & 15)) * D;
        else kr = SK + (((size_t)(kStageBlocks * l + (pos >> 4) - (kvl >> 4)) * nkv + g) * kBlock + (pos & 15)) * D;
        double a = 0.0;
        for (int i = 0; i < D; ++i) a += (double)q[i] * (double)kr[i];
        s = (float)(a * p.scale_log2);
      }
      const float mx = wave_max(s);
      const float mnew = fmaxf(mr, mx);
      if (mnew == -INFINITY) continue;
      const float alpha = exp2f(mr - mnew);
      const float pr = valid ? exp2f(s - mnew) : 0.f;
      double psum = pr;
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) psum += __shfl_xor(psum, mm);
      lr = lr * (double)alpha + psum;
      o0 *= alpha; o1 *= alpha;
      const int nval = min(64, we - p0);
      for (int t = 0; t < nval; ++t) {
        const double pt = __shfl(pr, t);
        const int vp = p0 + t;
        if (vp < lw) continue;   // below the window: weight 0, and its block may be released
        const float* vrow =
            vp < kvl ? Vp + ((size_t)clamp_blk(bt[vp >> 4], p.n_blocks) * nkv + g) * D * kBlock + (vp & 15)
                     : SV + ((size_t)(kStageBlocks * l + (vp >> 4) - (kvl >> 4)) * nkv + g) * D * kBlock + (vp & 15);
        if (lane < D) o0 += pt * (double)vrow[(size_t)lane * kBlock];
        if (lane + 64 < D) o1 += pt * (double)vrow[(size_t)(lane + 64) * kBlock];
      }
      mr = mnew;
    }
    float* dst = lds + ((size_t)wave * Mq + m) * PW;
    if (lane < D) dst[lane] = (float)o0;
    if (lane + 64 < D) dst[lane + 64] = (float)o1;
    if (lane == 0) { dst[D] = mr; dst[D + 1] = (float)lr; }
  }
  __syncthreads();
  float* out = p.part + (((size_t)l * nkv + g) * p.n_chunks + c) * 64 * PW;
  for (int idx = threadIdx.x; idx < Mq * D; idx += blockDim.x) {
    const int m = idx / D, dd = idx - m * D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds[((size_t)w * Mq + m) * PW + D]);
    double Oc = 0.0, Lc = 0.0;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float* src = lds + ((size_t)w * Mq + m) * PW;
        if (src[D] != -INFINITY) {
          const double f = exp2((double)src[D] - (double)M);
          Oc += (double)src[dd] * f;
          Lc += (double)src[D + 1] * f;
        }
      }
    }
    out[part_index(m, dd)] = (float)Oc;
    if (dd == 0) { out[part_index(m, D)] = M; out[part_index(m, D + 1)] = (float)Lc; }
  }
}

// Workgroups per (lane, kv head) of the bf16 kernel: the count that minimises
// (launch waves of one workgroup per CU) x (the longest range in 64-position stages
// at full capacity + the ring's fill, about 3 stages), within the block-id capacity of
// a workgroup.  Ties go to fewer ranges.
static int attn_ranges(const AttnParams& p) {
  const long pairs = (long)p.nkv * p.ri.L;
  // chunks a lane's rows can see: all of them, or with a window of W the at most
  // ceil((W + 15) / chunk) + 1 chunks that W - 1 + cols <= W + 15 positions touch
  const int nc = p.window > 0 ? std::min(p.n_chunks, (p.window + kMaxCols - 1 + p.chunk - 1) / p.chunk + 1)
                              : p.n_chunks;
  const long cap = p.window > 0 ? (long)nc * p.chunk : (long)p.max_blocks * kBlock;
  int best = nc;
  long best_cost = -1;
  for (int gx = 1; gx <= nc; ++gx) {
    const long per = (nc + gx - 1) / gx;
    if (per * (p.chunk / kBlock) > kAttnWgBlocks) continue;
    long longest = 0;
    for (int x = 0; x < gx; ++x) {
      const long c0 = (long)x * nc / gx, c1 = (long)(x + 1) * nc / gx;
      const long pos = std::min(c1 * p.chunk, cap) - c0 * p.chunk;
      longest = std::max(longest, (pos + 63) / 64);
    }
    const long cost = (pairs * gx + kCUs - 1) / kCUs * (longest + 3);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = gx; }
  }
  return best;
}

int launch_attention(const AttnParams& p, bool bf16, hipStream_t st) {
  dim3 block(256);
  if (bf16) {
    dim3 grid(attn_ranges(p), p.nkv, p.ri.L);
    hipLaunchKernelGGL(k_attn_bf16, grid, dim3(512), 0, st, p);
  } else {
    int maxMq = 0;
    for (int l = 0; l < p.ri.L; ++l) maxMq = p.ri.lane_cols[l] * p.G > maxMq ? p.ri.lane_cols[l] * p.G : maxMq;
    const size_t lds = (size_t)4 * maxMq * (p.d + kAttnPartPad) * sizeof(float);
    hipLaunchKernelGGL(k_attn_f32, dim3(p.n_chunks, p.nkv, p.ri.L), block, lds, st, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Merge the chunk partials of each (lane, kv head) in chunk order; write o = O / L.
// Thread = (query row m, four consecutive d), rows fastest: `rp` rows (a power of two
// covering the lane's queries) by 256 / rp four-float granules per workgroup, so a
// chunk's granule is read as one contiguous run.  Chunk loads are issued in batches of
// kCombineBatch before the float64 merge, which visits the chunks in order.
constexpr int kCombineBatch = 16;

template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnParams p, T* o, int rp) {
  const int g = blockIdx.x, l = blockIdx.y;
  const int D = p.d, PW = D + kAttnPartPad;
  const int m = threadIdx.x & (rp - 1), dq = blockIdx.z * (256 / rp) + threadIdx.x / rp;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int Mq = cols * p.G;
  if (m >= Mq || dq >= D / 4) return;
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int nch = min((end + p.chunk - 1) / p.chunk, p.n_chunks);
  const int cl = p.window > 0 ? max(0, kvl - p.window + 1) / p.chunk : 0;   // first chunk in any window
  const float* base = p.part + ((size_t)l * p.nkv + g) * p.n_chunks * 64 * PW;
  const size_t cstride = (size_t)64 * PW;
  const size_t io = part_index(m, 4 * dq), im = part_index(m, D);
  // one pass in chunk order with a running max M: acc = sum_c O_c 2^(m_c - M), rescaled
  // (in float64) whenever M grows
  double M = -INFINITY, Oc[4] = {0.0, 0.0, 0.0, 0.0}, Lc = 0.0;
  for (int c0 = cl; c0 < nch; c0 += kCombineBatch) {
    f32x4 ov[kCombineBatch];
    float mv[kCombineBatch], lv[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const float* src = base + (size_t)min(c0 + i, nch - 1) * cstride;
      ov[i] = *reinterpret_cast<const f32x4*>(src + io);
      const float2 ml = *reinterpret_cast<const float2*>(src + im);   // (max, sum): one load
      mv[i] = ml.x;
      lv[i] = ml.y;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) bm = fmaxf(bm, mv[i]);
    if ((double)bm > M) {
      const double r = M == -INFINITY ? 0.0 : exp2(M - (double)bm);
#pragma unroll
      for (int e = 0; e < 4; ++e) Oc[e] *= r;
      Lc *= r;
      M = bm;
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      if (c0 + i < nch && mv[i] != -INFINITY) {
        // the chunk's weight 2^(m_c - M) <= 1 by the hardware exp2 (float32; the float64
        // library call, once per thread and chunk, was most of the launch's arithmetic)
        const double f = (double)__builtin_amdgcn_exp2f((float)((double)mv[i] - M));
#pragma unroll
        for (int e = 0; e < 4; ++e) Oc[e] += (double)ov[i][e] * f;
        Lc += (double)lv[i] * f;
      }
    }
  }
  const int j = m / p.G, hh = m - j * p.G;
  const int K = p.nq * D;
  const size_t plane = act_plane(p.ri.R, K);
  const int k0 = (g * p.G + hh) * D + 4 * dq;
#pragma unroll
  for (int e = 0; e < 4; ++e) st_out(o, plane, act_index(o, rs + j, k0 + e, K), (float)(Oc[e] / Lc));
}

int launch_attn_combine(const AttnParams& p, void* o, bool bf16, hipStream_t st) {
  int maxMq = 0;
  for (int l = 0; l < p.ri.L; ++l) maxMq = p.ri.lane_cols[l] * p.G > maxMq ? p.ri.lane_cols[l] * p.G : maxMq;
  int rp = 1;
  while (rp < maxMq) rp *= 2;                 // maxMq <= 64
  const int gpw = 256 / rp;                   // granules per workgroup
  dim3 grid(p.nkv, p.ri.L, (p.d / 4 + gpw - 1) / gpw), block(256);
  if (bf16) hipLaunchKernelGGL(k_attn_combine<bf16_t>, grid, block, 0, st, p, reinterpret_cast<bf16_t*>(o), rp);
  else hipLaunchKernelGGL(k_attn_combine<float>, grid, block, 0, st, p, reinterpret_cast<float*>(o), rp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
