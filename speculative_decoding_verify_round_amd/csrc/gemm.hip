// Skinny-M projections and the fused LM head of the verify round (gfx950).
//
// A verify round multiplies at most 64 rows by every weight matrix of the
// model, so the pass is bound by streaming the weights from HBM once ("that
// pass is mostly the card streaming the weights from memory", "Speculative
// decoding", gpillon.github.io/ignis).  Both operands are stored as 1 KB MFMA
// fragments (frag_off), so every wave load is one contiguous 1 KB.
//
// Three cores share the fragment layout and the weight ring (an eight-step register
// ring per wave, non-temporal loads):
//  * R <= 16 (k_proj_direct): one wave per workgroup on two tiles, the activation
//    fragments read straight from memory into a ring beside the weights';
//  * R > 16 (k_proj_bal, proj_core_xw): eight waves with split roles -- main waves
//    own a unit (tile pair) each, two helpers share a fifth, two loaders copy the
//    activation chunks into an LDS ring by DMA;
//  * the LM head and the race (proj_core): four waves on T tiles each share a
//    double-buffered LDS ring of activation chunks; the X chunk for the next step
//    range is fetched at the start of a chunk and written to LDS at its end, so every
//    global load has a whole chunk of MFMA steps to arrive (the in-order vmcnt
//    counter never makes a step wait for a younger load).
//
// Numerics: each output element is one fp32 MFMA accumulation chain over its
// split in a fixed K order (per step the lo plane, then the hi plane); K
// splits depend on the matrix shape only and partials are summed in order by
// the consumer, so a row's result never depends on how many rows the round
// carries.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace sv {

constexpr int kUnit = 8;   // MFMA k-steps (32 each) per 256-wide unit; splits are whole units

template <int RT, int T, int XS, int KC, int NW = 4>
struct CoreShape {
  static constexpr int NC = kUnit / KC;      // X chunks per unit
  static constexpr int NB = KC * RT * XS;    // 1 KB X fragments per chunk
  static constexpr int NBW = (NB + NW - 1) / NW;   // staged per wave (NW waves per workgroup)
};

// acc[j][t] += W tile j (16 features) . X row tile t over the unit range
// [step0 / 8, step0 / 8 + nu).  wp[j] points at tile j's fragment of step
// step0, lane offset included; consecutive steps of a tile are wstep elements
// apart (weights are stored step-major).  xl: LDS ring [2][NB][64] u32x4.  Every wave of
// the workgroup must call this with the same step0 and nu.
template <int RT, int T, int XS, int KC, int NW = 4>
__device__ __forceinline__ void proj_core(const bf16_t* const (&wp)[T], size_t wstep, const bf16_t* __restrict__ X,
                                          size_t xplane, int KS, int step0, int nu, u32x4* xl,
                                          f32x4 (&acc)[T][RT]) {
  using C = CoreShape<RT, T, XS, KC, NW>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // this wave's share of an X chunk: fragment b = (plane * RT + tile) * KC + step
  // (with NB not a multiple of NW the last waves stage fewer; the test is wave-uniform)
  uint32_t xoff[C::NBW];
#pragma unroll
  for (int i = 0; i < C::NBW; ++i) {
    const int b = min(wave * C::NBW + i, C::NB - 1);
    const int pl = b / (RT * KC), t = (b / KC) % RT, st = b % KC;
    xoff[i] = (uint32_t)(pl * xplane + ((size_t)t * KS + st) * 512 + lane * 8);
  }
  u32x4 sx[C::NBW];
  auto stage_load = [&](int stepc) {
#pragma unroll
    for (int i = 0; i < C::NBW; ++i)
      if (C::NB % NW == 0 || wave * C::NBW + i < C::NB)
        sx[i] = *reinterpret_cast<const u32x4*>(X + xoff[i] + (size_t)stepc * 512);
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::NBW; ++i)
      if (C::NB % NW == 0 || wave * C::NBW + i < C::NB)
        xl[((size_t)buf * C::NB + wave * C::NBW + i) * 64 + lane] = sx[i];
  };
  u32x4 wr[kUnit][T];
  stage_load(step0);
#pragma unroll
  for (int k = 0; k < kUnit; ++k)
#pragma unroll
    for (int j = 0; j < T; ++j) wr[k][j] = ld_stream(reinterpret_cast<const u32x4*>(wp[j] + (size_t)k * wstep));
  stage_store(0);
  __syncthreads();
  int cb = 0;
  auto run_unit = [&](auto more_tag, int u) {
    constexpr bool MORE = decltype(more_tag)::value;
#pragma unroll
    for (int h = 0; h < C::NC; ++h) {
      const bool next = (h + 1 < C::NC) || MORE;
      if (next) stage_load(step0 + u * kUnit + (h + 1) * KC);
      // keep the issue order as written: the scheduler would otherwise sink the
      // prefetches next to their first use and expose the full memory latency
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < KC; ++st) {
        const int k = h * KC + st;
        u32x4 xo[XS][RT];
#pragma unroll
        for (int pl = 0; pl < XS; ++pl)
#pragma unroll
          for (int t = 0; t < RT; ++t) xo[pl][t] = xl[((size_t)cb * C::NB + (pl * RT + t) * KC + st) * 64 + lane];
#pragma unroll
        for (int j = 0; j < T; ++j)
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int pl = XS - 1; pl >= 0; --pl) acc[j][t] = mfma_bf16(wr[k][j], xo[pl][t], acc[j][t]);
        if constexpr (MORE) {
#pragma unroll
          for (int j = 0; j < T; ++j)
            wr[k][j] = ld_stream(reinterpret_cast<const u32x4*>(wp[j] + (size_t)((u + 1) * kUnit + k) * wstep));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (next) stage_store(cb ^ 1);
      __syncthreads();
      cb ^= 1;
    }
  };
  for (int u = 0; u + 1 < nu; ++u) run_unit(std::true_type{}, u);
  run_unit(std::false_type{}, nu - 1);
}

// R > 16, split roles in an eight-wave workgroup of up to five units:
//  * main waves 0..3 own units 0..3: they stream their unit's weights and run its MFMAs
//    for every row tile;
//  * helper waves 4, 5 share a fifth unit: helper h runs its MFMAs for row tiles h and
//    h + 2 only (both load the unit's weights, the second from L2), so no SIMD carries
//    two full units -- waves w and w + 4 share a SIMD, and of two MFMA-heavy waves on
//    one SIMD the younger is starved of MFMA issue until the older one ends;
//  * loader waves 6, 7 copy X chunks into a kXSlots-deep LDS ring by DMA.
// Each wave's in-order vmcnt counter then holds one kind of load: the compute waves
// never wait for an X load behind their weights, so their weight ring runs a whole
// unit (eight steps) ahead, and the loaders keep the X ring kXSlots - 1 chunks ahead.
// One workgroup barrier per chunk publishes it (and frees the slot the previous chunk
// used); it waits for LDS accesses only.  (A two-unit weight ring measured slower:
// four compute waves with eight steps of 2 KB in flight each already cover the memory
// latency, and the deeper ring only adds registers.)
constexpr int kXSlots = 4;
constexpr int kXWaves = 2;
constexpr int kMainWaves = 4;
constexpr int kHelpers = 2;
constexpr int kMaxUnits = kMainWaves + 1;   // units per workgroup

// ------------------------------------------------------------------------------- cut units
// A gate/up launch whose unit count is not a multiple of the CU count would leave some
// CUs one whole unit more to stream than the others (1088 units: 64 CUs with five, 192
// with four), and the launch lasts as long as its busiest CU.  The balanced launch gives
// every CU `base` whole units plus one K piece (whole 256-wide steps) of one of the `rem`
// units left over, each of those cut into `pq` pieces, so every CU streams the same
// weight bytes to within a piece.  A piece's gate and up sums go to Q with
// agent-coherent stores (sc1: they reach the point of coherence of all CUs before the
// wave's store counter drops); once they are complete, the wave (or workgroup) counts
// itself in with an atomic add, and the one that completes the unit's count reads the
// pieces back with sc1 loads, adds them in piece order in float64, applies the SwiGLU
// epilogue and zeroes the counter for the next launch.  Pieces and their order follow
// from the shape alone, so a row's result never depends on how many rows the round has.
constexpr int kMaxPieces = 4;

// float(silu(g) * u) evaluated in float64 from the fp32 projections
__device__ __forceinline__ float swiglu(float g32, float u32) {
  const double g = (double)g32, u = (double)u32;
  return (float)(g / (1.0 + exp(-g)) * u);
}

struct SwigluPlan {
  int base, rem, pq;
};

__host__ __device__ inline SwigluPlan swiglu_plan(int units, int K) {
  SwigluPlan s{units / kCUs, units % kCUs, 0};
  const int U = K >> 8;
  if (s.base < 1 || s.base > kMainWaves || s.rem == 0) return SwigluPlan{s.base, 0, 0};
  s.pq = kCUs / s.rem;
  s.pq = s.pq < U ? s.pq : U;
  s.pq = s.pq < kMaxPieces ? s.pq : kMaxPieces;
  if (s.pq < 2) return SwigluPlan{s.base, 0, 0};   // nothing to even out
  return s;
}

int swiglu_pieces(int N, int K, int* rem, int* pq) {
  const SwigluPlan s = swiglu_plan((N + 15) / 16, K);
  *rem = s.rem;
  *pq = s.pq;
  return s.rem * s.pq;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t piece_rsrc(const ProjParams& p) {
  const int bytes = p.rem * p.pq * 2 * p.R * 16 * 4;
  return __builtin_amdgcn_make_buffer_rsrc(p.Q, 0, bytes, 0x00020000);
}

// Byte offset of Q[r][part][j][row][f].
__device__ __forceinline__ uint32_t piece_off(const ProjParams& p, int r, int part, int j, int row, int f) {
  return (uint32_t)((((((size_t)r * p.pq + part) * 2 + j) * p.R + row) * 16 + f) * 4);
}

// Row tile t of tile j (gate 0, up 1) of a piece: lane holds features 4 kq .. + 3 of row
// 16 t + r16.
__device__ __forceinline__ void piece_store(const ProjParams& p, __amdgpu_buffer_rsrc_t rs, int r, int part, int t,
                                            int j, f32x4 v) {
  const int lane = threadIdx.x & 63, row = 16 * t + (lane & 15);
  if (row >= p.R) return;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, piece_off(p, r, part, j, row, 4 * (lane >> 4)),
                                         0, 16);
}

// The pieces of one (row, four features) item of cut unit r: gate and up, pq of each
// (slots past pq repeat the last piece and are not added).
struct PieceLoads {
  u32x4 g[kMaxPieces], u[kMaxPieces];
};

__device__ __forceinline__ PieceLoads piece_load(const ProjParams& p, __amdgpu_buffer_rsrc_t rs, int r, int item) {
  const int row = item >> 2, f = 4 * (item & 3);
  PieceLoads ld;
#pragma unroll
  for (int q = 0; q < kMaxPieces; ++q) {
    const int qc = min(q, p.pq - 1);
    ld.g[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, piece_off(p, r, qc, 0, row, f), 0, 16);
    ld.u[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, piece_off(p, r, qc, 1, row, f), 0, 16);
  }
  return ld;
}

// Adds the pieces in piece order in float64 and stores the item's SwiGLU output.
__device__ __forceinline__ void piece_finish(const ProjParams& p, int unit, int item, const PieceLoads& ld) {
  const int row = item >> 2, f = 4 * (item & 3);
  double gs[4], us[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gs[e] = (double)__uint_as_float(ld.g[0][e]);
    us[e] = (double)__uint_as_float(ld.u[0][e]);
  }
#pragma unroll
  for (int q = 1; q < kMaxPieces; ++q) {
    if (q >= p.pq) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gs[e] += (double)__uint_as_float(ld.g[q][e]);
      us[e] += (double)__uint_as_float(ld.u[q][e]);
    }
  }
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = swiglu((float)gs[e], (float)us[e]);
  const int nf = unit * 16 + f;
  if (nf + 4 <= p.N) st_out4(p.Y, p.yplane, row, nf, p.N, v);
}

// Loader waves: X chunk g of the unit range into ring slot g % kXSlots, then the
// chunk's barrier once it has landed.
template <int RT, int XS, int KC>
// rs, SK: the chunks start at step rs of a range of SK steps and wrap around (rs = 0: in
// order).
__device__ __forceinline__ void x_loader(const bf16_t* __restrict__ X, size_t xplane, int KS, int step0, int nu,
                                         char* xring, int lw, int rs = 0, int SK = 1 << 30) {
  constexpr int NB = KC * RT * XS;           // 1 KB X fragments per chunk: b = (plane * RT + tile) * KC + step
  constexpr int NC = kUnit / KC;             // chunks per unit
  constexpr int CHUNK = NB * 1024;
  constexpr int PER = NB / kXWaves;          // DMAs per loader wave per chunk
  static_assert(NB % kXWaves == 0 && (NC == 1 || NC == 2), "chunk shape");
  const int lane = threadIdx.x & 63;
  const int G = nu * NC;
  auto issue = [&](int g) {
    char* slot = xring + (g % kXSlots) * CHUNK;
    int gk = g * KC + rs;
    gk = gk < SK ? gk : gk - SK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = lw + kXWaves * i;
      const int pl = b / (RT * KC), t = (b / KC) % RT, st = b % KC;
      const bf16_t* src = X + pl * xplane + ((size_t)t * KS + step0 + gk + st) * 512;
      dma16<false>(src, lane * 16, slot + b * 1024);
    }
  };
  for (int g = 0; g < kXSlots - 1 && g < G; ++g) issue(g);
  for (int g = 0; g < G; ++g) {
    const int after = min(G - 1, g + kXSlots - 2) - g;   // chunks issued after g
    if (after >= 2) wait_vm<2 * PER>();
    else if (after == 1) wait_vm<PER>();
    else wait_vm<0>();
    wg_barrier();                                        // chunk g is in LDS
    if (g + kXSlots - 1 < G) issue(g + kXSlots - 1);     // into the slot chunk g - 1 used
  }
}

// Compute waves: acc[j][i] += W tile j . X row tile rt(i) over the unit range, i < NR,
// with row tile rt(i) = r0 + RS i (main waves: r0 = 0, RS = 1, NR = RT; helpers:
// r0 = h, RS = 2, NR = 2, a row tile past RT reads a valid slot and is discarded).
// NT: non-temporal weight loads (data read once); helpers share a unit and load it
// cacheable so that the second one finds it in L2.
// g0: chunks of the launch before the range: the range's first weights are requested
// before the wave passes those chunks' barriers.  rs, SK: the steps start at step rs of
// SK and wrap around, as the X chunks do (rs = 0: in order).
template <int RT, int T, int XS, int KC, int NR, bool NT>
__device__ __forceinline__ void proj_core_xw(const bf16_t* const (&wp)[T], size_t wstep, int r0, int RS, int nu,
                                             const char* xring, f32x4 (&acc)[T][NR], int g0 = 0, int rs = 0,
                                             int SK = 1 << 30) {
  constexpr int NB = KC * RT * XS;
  constexpr int NC = kUnit / KC;
  constexpr int CHUNK = NB * 1024;
  const int lane = threadIdx.x & 63;
  int rt[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) rt[i] = min(r0 + RS * i, RT - 1);
  // weight ring over one unit: slot k holds step k of the current unit; a unit with
  // MORE refills each slot with the next unit's step once its MFMAs have read it.  The
  // loads sit on straight-line paths, so the compiler's waits are exact.
  u32x4 wr[kUnit][T];
  auto load = [&](int slot, int step) {
    step += rs;
    step = step < SK ? step : step - SK;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const u32x4* src = reinterpret_cast<const u32x4*>(wp[j] + (size_t)step * wstep);
      wr[slot][j] = NT ? ld_stream(src) : *src;
    }
  };
  auto run_unit = [&](auto more_tag, int u) {
    constexpr bool MORE = decltype(more_tag)::value;
    auto chunk = [&](auto h_tag) {
      constexpr int h = decltype(h_tag)::value;
      const int g = g0 + u * NC + h;
      wg_barrier();                                        // chunk g is in LDS
      const char* slot = xring + (g % kXSlots) * CHUNK + lane * 16;
#pragma unroll
      for (int st = 0; st < KC; ++st) {
        const int k = h * KC + st;
        u32x4 xo[XS][NR];
#pragma unroll
        for (int pl = 0; pl < XS; ++pl)
#pragma unroll
          for (int i = 0; i < NR; ++i)
            xo[pl][i] = *reinterpret_cast<const u32x4*>(slot + ((pl * RT + rt[i]) * KC + st) * 1024);
#pragma unroll
        for (int j = 0; j < T; ++j)
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int pl = XS - 1; pl >= 0; --pl)
              acc[j][i] = mfma_bf16(wr[k][j], xo[pl][i], acc[j][i]);
        if constexpr (MORE) load(k, (u + 1) * kUnit + k);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    chunk(std::integral_constant<int, 0>{});
    if constexpr (NC == 2) chunk(std::integral_constant<int, 1>{});
  };
#pragma unroll
  for (int k = 0; k < kUnit; ++k) load(k, k);
  for (int g = 0; g < g0; ++g) wg_barrier();
  for (int u = 0; u + 1 < nu; ++u) run_unit(std::true_type{}, u);
  run_unit(std::false_type{}, nu - 1);
}

// One row tile (R <= 16), one wave per workgroup: the activation fragments are
// read straight from memory (they stay in L2) into a ring of the same depth as
// the weights', so the launch can carry four times as many workgroups (the
// dispatcher balances them across CUs) and needs neither LDS nor barriers.
template <int T, int XS>
__device__ __forceinline__ void proj_core_direct(const bf16_t* const (&wp)[T], size_t wstep,
                                                 const bf16_t* __restrict__ X, size_t xplane, int step0, int nu,
                                                 int rows, f32x4 (&acc)[T], int rs = 0, int SK = 1 << 30) {
  const int lane = threadIdx.x & 63;
  const bf16_t* xp = X + (size_t)step0 * 512 + lane * 8;   // row tile 0: fragment s at s * 512
  // lane i carries row i % 16 of an X fragment: lanes of the tile's padding rows
  // (zeros) load nothing, so a round of R < 16 rows reads R / 16 of every fragment
  const bool xrow = (lane & 15) < rows;
  u32x4 wr[kUnit][T], xr[kUnit][XS];
  auto load = [&](int slot, int st) {
    st += rs;
    st = st < SK ? st : st - SK;
#pragma unroll
    for (int pl = 0; pl < XS; ++pl) {
      xr[slot][pl] = u32x4{0u, 0u, 0u, 0u};
      if (xrow) xr[slot][pl] = *reinterpret_cast<const u32x4*>(xp + pl * xplane + (size_t)st * 512);
    }
#pragma unroll
    for (int j = 0; j < T; ++j) wr[slot][j] = ld_stream(reinterpret_cast<const u32x4*>(wp[j] + (size_t)st * wstep));
  };
#pragma unroll
  for (int k = 0; k < kUnit; ++k) load(k, k);
  auto run_unit = [&](auto more_tag, int u) {
    constexpr bool MORE = decltype(more_tag)::value;
#pragma unroll
    for (int k = 0; k < kUnit; ++k) {
#pragma unroll
      for (int j = 0; j < T; ++j)
#pragma unroll
        for (int pl = XS - 1; pl >= 0; --pl) acc[j] = mfma_bf16(wr[k][j], xr[k][pl], acc[j]);
      if constexpr (MORE) load(k, (u + 1) * kUnit + k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int u = 0; u + 1 < nu; ++u) run_unit(std::true_type{}, u);
  run_unit(std::false_type{}, nu - 1);
}

template <int RT>
constexpr int chunk_steps() { return RT <= 2 ? 8 : 4; }


// ------------------------------------------------------------------------------- projection
// R > 16: at most 256 workgroups of eight waves per launch; workgroup b takes split
// s = b / cols and part w = b % cols of it.  Plain outputs (EPI 0) are dealt by
// 16-feature tile: tiles [w N_t / cols, (w + 1) N_t / cols), at most eight, two per main
// wave, so the busiest CU streams at most one tile more than the others (448 QKV tiles
// at four splits: seven per workgroup, where tile pairs would give half of them eight).
// SwiGLU outputs (EPI 1) are dealt by unit (gate and up tile u): units [w P / cols,
// (w + 1) P / cols), at most five, units 0..3 to the main waves and a fifth to the two
// helpers (1088 gate/up pairs become 4 or 5 per CU, where whole 4-pair workgroups leave
// 16 CUs with twice the work).
template <int RT, int XS, int EPI, int NR>
__device__ __forceinline__ void bal_epilogue(const ProjParams& p, const int (&tile)[2], int s, int r0, int RS,
                                             const f32x4 (&acc)[2][NR]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, kq = lane >> 4;
  // lane holds D[feature 16 tile + 4 kq + e][row 16 rt + r16]
  if constexpr (EPI == 0) {
    const bool vec = (p.N & 3) == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (tile[j] >= p.tiles) continue;
      const int nf = tile[j] * 16 + 4 * kq;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int t = r0 + RS * i;
        const int r = t * 16 + r16;
        if (t >= RT || r >= p.R) continue;
        float* dst = p.P + ((size_t)s * p.R + r) * p.N + nf;
        if (vec && nf + 4 <= p.N) {
          *reinterpret_cast<f32x4*>(dst) = acc[j][i];
        } else {
          for (int e = 0; e < 4 && nf + e < p.N; ++e) dst[e] = acc[j][i][e];
        }
      }
    }
  } else {
    if (tile[0] >= p.tiles) return;
    const int nf = tile[0] * 16 + 4 * kq;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int t = r0 + RS * i;
      const int r = t * 16 + r16;
      if (t >= RT || r >= p.R || nf + 4 > p.N) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = swiglu(acc[0][i][e], acc[1][i][e]);
      st_out4(p.Y, p.yplane, r, nf, p.N, v);
    }
  }
}

// K rotation of whole unit `unit` in a balanced SwiGLU launch: every workgroup (and
// every wave-sized workgroup of the same unit in the one-row-tile launch) takes the K
// steps from the start of its piece on, wrapping around, so the pieces are done first.
__device__ __forceinline__ int cut_rotation(const ProjParams& p, int unit) {
  const int w = unit / p.base, U = p.K >> 8;
  if (w >= p.rem * p.pq) return 0;
  return (w % p.pq) * U / p.pq;
}

// Balanced SwiGLU launch, one workgroup per CU (S = 1), K order rotated to start at the
// workgroup's piece: main wave i < base streams whole unit base w + i; helper 0
// computes piece w (if any) over all row tiles from the same X chunks, stores it, and
// over the next chunk barriers lets the stores complete, counts itself in, and -- if it
// completes the unit -- adds the pieces and writes the unit's SwiGLU output, so none of
// this lands on the launch's tail.  Every wave passes the same barriers.
template <int RT, int XS>
__device__ __forceinline__ void bal_cut(const ProjParams& p, char* xring) {
  constexpr int KC = chunk_steps<RT>(), T = 2, NC = kUnit / KC;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int w = blockIdx.x;
  const int KS = p.K >> 5, U = p.K >> 8, G = U * NC, SK = U * kUnit;
  const bool cut = w < p.rem * p.pq;
  const int r = w / p.pq, part = w - r * p.pq;
  const int k0 = cut ? part * U / p.pq : 0, k1 = cut ? (part + 1) * U / p.pq : 0;
  const int rs = k0 * kUnit;
  if (wave >= kMainWaves + kHelpers) {
    x_loader<RT, XS, KC>(p.X, p.xplane, KS, 0, U, xring, wave - kMainWaves - kHelpers, rs, SK);
    return;
  }
  if (wave < kMainWaves) {
    if (wave < p.base) {
      const int unit = w * p.base + wave;
      int tile[T] = {unit, unit};
      const bf16_t* wp[T] = {p.W0 + (size_t)unit * KS * 512 + lane * 8, p.W1 + (size_t)unit * KS * 512 + lane * 8};
      f32x4 acc[T][RT];
#pragma unroll
      for (int j = 0; j < T; ++j)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      proj_core_xw<RT, T, XS, KC, RT, true>(wp, 512, 0, 1, U, xring, acc, 0, rs, SK);
      bal_epilogue<RT, XS, 1, RT>(p, tile, 0, 0, 1, acc);
    } else {
      for (int g = 0; g < G; ++g) wg_barrier();
    }
    return;
  }
  if (wave != kMainWaves || !cut) {
    for (int g = 0; g < G; ++g) wg_barrier();
    return;
  }
  // helper 0: the piece, chunks 0 .. (k1 - k0) NC - 1 of the rotated order
  const int unit = p.base * kCUs + r;
  const size_t off = ((size_t)unit * KS + (size_t)k0 * kUnit) * 512 + lane * 8;
  const bf16_t* wp[T] = {p.W0 + off, p.W1 + off};
  f32x4 acc[T][RT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  proj_core_xw<RT, T, XS, KC, RT, true>(wp, 512, 0, 1, k1 - k0, xring, acc);
  const auto rsrc = piece_rsrc(p);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < T; ++j) piece_store(p, rsrc, r, part, t, j, acc[j][t]);
  int g = (k1 - k0) * NC;
  auto pass = [&](int n) {   // n chunk barriers, or as many as are left
    for (int i = 0; i < n && g < G; ++i, ++g) wg_barrier();
  };
  pass(2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the piece is stored
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pass(2);
  if (__builtin_amdgcn_readfirstlane(old) == p.pq - 1) {
    // this piece completed the unit: two (row, four features) items per lane at a time,
    // loads issued one chunk barrier before their use
    for (int it0 = 0; it0 < p.R * 4; it0 += 128) {
      PieceLoads ld[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) ld[i] = piece_load(p, rsrc, r, min(it0 + 64 * i + lane, p.R * 4 - 1));
      pass(1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (it0 + 64 * i + lane < p.R * 4) piece_finish(p, unit, it0 + 64 * i + lane, ld[i]);
    }
    if (lane == 0) __hip_atomic_store(p.cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  pass(G);
}

template <int RT, int XS, int EPI>
__global__ __launch_bounds__(512, 1) void k_proj_bal(ProjParams p) {
  constexpr int KC = chunk_steps<RT>(), T = 2;
  __shared__ __attribute__((aligned(1024))) char xring[kXSlots * KC * RT * XS * 1024];
  if constexpr (EPI == 1) {
    if (p.rem > 0) {
      bal_cut<RT, XS>(p, xring);
      return;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // workgroup -> (split s, part w of cols): plain launches give each split its own count
  int s, w, cols;
  if constexpr (EPI == 0) {
    s = 0;
    w = blockIdx.x;
    cols = p.scols[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      if (i < p.S && w >= cols) {
        w -= cols;
        s = i;
        cols = p.scols[i];
      }
    }
  } else {
    s = blockIdx.x / p.cols;
    w = blockIdx.x % p.cols;
    cols = p.cols;
  }
  const int KS = p.K >> 5, U = p.K >> 8;
  const int u0 = (int)((long long)s * U / p.S), u1 = (int)((long long)(s + 1) * U / p.S);
  if (wave >= kMainWaves + kHelpers) {
    x_loader<RT, XS, KC>(p.X, p.xplane, KS, u0 * kUnit, u1 - u0, xring, wave - kMainWaves - kHelpers);
    return;
  }
  const bool helper = wave >= kMainWaves;
  // EPI 0: workgroup w of a split takes the 16-feature tiles [w tiles / cols, (w + 1) tiles /
  // cols), at most 2 kMainWaves of them, two per main wave in order (the last busy wave may
  // hold one); the helpers have none.  EPI 1: units (gate and up tile u) as listed above.
  int t0, nt;
  if constexpr (EPI == 0) {
    const int tb = (int)((long long)w * p.tiles / cols), te = (int)((long long)(w + 1) * p.tiles / cols);
    t0 = tb + 2 * wave;
    nt = helper ? 0 : max(0, min(2, te - t0));
  } else {
    const int ub = (int)((long long)w * p.units / cols), ue = (int)((long long)(w + 1) * p.units / cols);
    t0 = helper ? ub + kMainWaves : ub + wave;
    nt = t0 < ue ? 2 : 0;
  }
  if (nt == 0) {   // nothing to stream: keep the barrier count
    for (int g = 0; g < (u1 - u0) * (kUnit / KC); ++g) wg_barrier();
    return;
  }
  int tile[T];
  const bf16_t* wp[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    tile[j] = EPI == 1 ? t0 : t0 + j;
    const int tc = min(tile[j], p.tiles - 1);
    const bf16_t* base = (EPI == 1 && j == 1) ? p.W1 : p.W0;
    wp[j] = base + ((size_t)tc * KS + (size_t)u0 * kUnit) * 512 + lane * 8;
  }
  if constexpr (EPI == 0) {
    if (nt == 1) {   // one tile: its own chain, the second output slot skipped
      const bf16_t* wp1[1] = {wp[0]};
      f32x4 acc1[1][RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) acc1[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      proj_core_xw<RT, 1, XS, KC, RT, true>(wp1, 512, 0, 1, u1 - u0, xring, acc1);
      f32x4 acc[T][RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        acc[0][t] = acc1[0][t];
        acc[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const int tile1[T] = {tile[0], p.tiles};
      bal_epilogue<RT, XS, EPI, RT>(p, tile1, s, 0, 1, acc);
      return;
    }
  }
  if (!helper) {
    f32x4 acc[T][RT];
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    proj_core_xw<RT, T, XS, KC, RT, true>(wp, 512, 0, 1, u1 - u0, xring, acc);
    bal_epilogue<RT, XS, EPI, RT>(p, tile, s, 0, 1, acc);
  } else {
    const int h = wave - kMainWaves;
    f32x4 acc[T][2];
#pragma unroll
    for (int j = 0; j < T; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    proj_core_xw<RT, T, XS, KC, 2, false>(wp, 512, h, 2, u1 - u0, xring, acc);
    bal_epilogue<RT, XS, EPI, 2>(p, tile, s, h, 2, acc);
  }
}

// A piece of a cut unit, one wave: the unit's gate and up tiles over the piece's K range.
template <int XS>
__device__ __forceinline__ void direct_piece(const ProjParams& p) {
  const int lane = threadIdx.x & 63;
  const int pi = blockIdx.x - p.base * kCUs, r = pi / p.pq, part = pi - r * p.pq;
  const int unit = p.base * kCUs + r;
  const int KS = p.K >> 5, U = p.K >> 8;
  const int k0 = part * U / p.pq, k1 = (part + 1) * U / p.pq;
  const size_t off = ((size_t)unit * KS + (size_t)k0 * kUnit) * 512 + lane * 8;
  const bf16_t* wp[2] = {p.W0 + off, p.W1 + off};
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  proj_core_direct<2, XS>(wp, 512, p.X, p.xplane, k0 * kUnit, k1 - k0, p.R, acc);
  const auto rs = piece_rsrc(p);
  piece_store(p, rs, r, part, 0, 0, acc[0]);
  piece_store(p, rs, r, part, 0, 1, acc[1]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the piece is stored
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__builtin_amdgcn_readfirstlane(old) == p.pq - 1) {   // this piece completed the unit
    const int item = min(lane, p.R * 4 - 1);                 // R <= 16: one item per lane
    const PieceLoads ld = piece_load(p, rs, r, item);
    if (lane < p.R * 4) piece_finish(p, unit, lane, ld);
    if (lane == 0) __hip_atomic_store(p.cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// R <= 16: one wave per workgroup (T tiles, one split), epilogues as k_proj.  A
// balanced SwiGLU launch appends the piece workgroups after the whole units.
template <int T, int XS, int EPI>
__global__ __launch_bounds__(64) void k_proj_direct(ProjParams p) {
  if constexpr (EPI == 1) {
    if (p.rem > 0 && (int)blockIdx.x >= p.base * kCUs) {
      direct_piece<XS>(p);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x % p.cols, s = blockIdx.x / p.cols;
  const int KS = p.K >> 5, U = p.K >> 8;
  const int u0 = (int)((long long)s * U / p.S), u1 = (int)((long long)(s + 1) * U / p.S);
  int tile[T];
  const bf16_t* wp[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    tile[j] = EPI == 1 ? col : col * T + j;
    const int tc = min(tile[j], p.tiles - 1);
    const bf16_t* base = (EPI == 1 && j == 1) ? p.W1 : p.W0;
    wp[j] = base + ((size_t)tc * KS + (size_t)u0 * kUnit) * 512 + lane * 8;
  }
  f32x4 acc[T];
#pragma unroll
  for (int j = 0; j < T; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int rs = 0;
  if constexpr (EPI == 1)
    if (p.rem > 0) rs = cut_rotation(p, col) * kUnit;   // the K order of the unit's balanced workgroup
  proj_core_direct<T, XS>(wp, 512, p.X, p.xplane, u0 * kUnit, u1 - u0, p.R, acc, rs, U * kUnit);
  const int r = lane & 15, kq = lane >> 4;
  if (r >= p.R) return;
  if constexpr (EPI == 0) {
    const bool vec = (p.N & 3) == 0;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (tile[j] >= p.tiles) continue;
      const int nf = tile[j] * 16 + 4 * kq;
      float* dst = p.P + ((size_t)s * p.R + r) * p.N + nf;
      if (vec && nf + 4 <= p.N) {
        *reinterpret_cast<f32x4*>(dst) = acc[j];
      } else {
        for (int e = 0; e < 4 && nf + e < p.N; ++e) dst[e] = acc[j][e];
      }
    }
  } else {
    if (tile[0] >= p.tiles) return;
    const int nf = tile[0] * 16 + 4 * kq;
    if (nf + 4 <= p.N) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = swiglu(acc[0][e], acc[1][e]);
      st_out4(p.Y, p.yplane, r, nf, p.N, v);
    }
  }
}

// Workgroups per split of the balanced SwiGLU launch (at most 256 per launch, at most
// kMaxUnits units each).
static int bal_cols(int units, int S) {
  int cols = std::min(kCUs / S, units);
  if ((units + cols - 1) / cols > kMaxUnits) cols = (units + kMaxUnits - 1) / kMaxUnits;
  return std::max(cols, 1);
}

// Workgroups per split of a balanced plain launch: kCUs / S, or fewer when there are fewer
// tiles, or more when a workgroup would otherwise hold more than two tiles per main wave.
static int tile_cols(int tiles, int S) {
  int cols = std::min(kCUs / S, tiles);
  if ((tiles + cols - 1) / cols > 2 * kMainWaves) cols = (tiles + 2 * kMainWaves - 1) / (2 * kMainWaves);
  return std::max(cols, 1);
}

// Workgroups of each split of a balanced plain launch (returns their sum, the grid).  The
// splits of U units over S hold U / S units or one more, and a workgroup streams its units
// x (its tiles x 16 x 256 x 2 weight bytes + 64 x 256 x 4 activation bytes at 64 rows, those
// L2 hits holding the read window about a quarter as long): units x (tiles + 2.24) in tile
// equivalents.  A split of more units gets more workgroups when that lowers the largest
// such cost within kCUs workgroups of at most 2 kMainWaves tiles (six splits of 11 or 12
// units over 320 tiles: 40 workgroups of eight tiles for an 11-unit split, 46 of seven for
// a 12-unit one, where 42 each give the 12-unit splits eight); otherwise every split gets
// tile_cols workgroups.
static int plan_cols(int tiles, int S, int U, int (&scols)[8]) {
  constexpr double kAct = 2.24;
  int us[8];
  for (int s = 0; s < S; ++s) us[s] = (s + 1) * U / S - s * U / S;
  const int uc = tile_cols(tiles, S), ut = (tiles + uc - 1) / uc;
  double uniform = 0.0;
  for (int s = 0; s < S; ++s) uniform = std::max(uniform, us[s] * (ut + kAct));
  auto tiles_for = [&](int u, double c) {   // most tiles a workgroup of u units may take at cost c
    int t = 2 * kMainWaves;
    while (t >= 1 && u * (t + kAct) > c + 1e-9) --t;
    return t;
  };
  double best = uniform;
  bool found = false;
  for (int s0 = 0; s0 < S; ++s0)
    for (int t0 = 1; t0 <= 2 * kMainWaves; ++t0) {
      const double c = us[s0] * (t0 + kAct);
      if (c >= best - 1e-9) continue;
      int total = 0;
      for (int s = 0; s < S && total <= kCUs; ++s) {
        const int t = tiles_for(us[s], c);
        total = t < 1 ? kCUs + 1 : total + (tiles + t - 1) / t;
      }
      if (total <= kCUs) {
        best = c;
        found = true;
      }
    }
  int grid = 0;
  for (int s = 0; s < 8; ++s) {
    scols[s] = s >= S ? 0 : found ? (tiles + tiles_for(us[s], best) - 1) / tiles_for(us[s], best) : uc;
    grid += scols[s];
  }
  return grid;
}

int launch_proj(const ProjParams& p0, bool swiglu, int xs, hipStream_t st) {
  ProjParams p = p0;
  const int RT = (p.R + 15) / 16;
  p.rem = 0;
  if (swiglu && p.S == 1 && p.Q && p.cnt) {
    const SwigluPlan sp = swiglu_plan(p.tiles, p.K);
    p.base = sp.base; p.rem = sp.rem; p.pq = sp.pq;
  }
  if (RT == 1) {   // one wave per workgroup, two tiles per wave
    constexpr int T = 2;
    p.cols = swiglu ? p.tiles : (p.tiles + T - 1) / T;
    dim3 grid(p.rem ? p.base * kCUs + p.rem * p.pq : p.cols * p.S), block(64);
    if (swiglu) hipLaunchKernelGGL((k_proj_direct<2, 2, 1>), grid, block, 0, st, p);
    else if (xs == 2) hipLaunchKernelGGL((k_proj_direct<2, 2, 0>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_proj_direct<2, 1, 0>), grid, block, 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  p.units = swiglu ? p.tiles : (p.tiles + 1) / 2;
  int nwg;
  if (swiglu) {
    p.cols = bal_cols(p.units, p.S);
    nwg = p.rem ? kCUs : p.cols * p.S;
  } else {
    nwg = plan_cols(p.tiles, p.S, p.K >> 8, p.scols);
  }
  dim3 grid(nwg), block(512);
#define SV_P(RT_, XS_, E_) hipLaunchKernelGGL((k_proj_bal<RT_, XS_, E_>), grid, block, 0, st, p)
#define SV_P_RT(XS_, E_)             \
  switch (RT) {                      \
    case 2: SV_P(2, XS_, E_); break; \
    case 3: SV_P(3, XS_, E_); break; \
    default: SV_P(4, XS_, E_); break; \
  }
  if (swiglu) {
    SV_P_RT(2, 1);
  } else if (xs == 2) {
    SV_P_RT(2, 0);
  } else {
    SV_P_RT(1, 0);
  }
#undef SV_P_RT
#undef SV_P
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// fp32 weights: a plain VALU dot product per output (fixed K order).
__global__ void k_gemm_f32(GemmF32Params p, int use_swiglu) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x, r = blockIdx.y;
  if (n >= p.N) return;
  const float* x = p.X + (size_t)r * p.K;
  const float* w = p.W0 + (size_t)n * p.K;
  double a = 0.0;
  for (int k = 0; k < p.K; ++k) a += (double)x[k] * (double)w[k];
  if (!use_swiglu) {
    p.P[(size_t)r * p.N + n] = (float)a;
  } else {
    const float* w1 = p.W1 + (size_t)n * p.K;
    double b = 0.0;
    for (int k = 0; k < p.K; ++k) b += (double)x[k] * (double)w1[k];
    p.Ya[(size_t)r * p.N + n] = swiglu((float)a, (float)b);
  }
}

int launch_gemm_f32(const GemmF32Params& p, bool swiglu, hipStream_t st) {
  dim3 grid((p.N + 255) / 256, p.R), block(256);
  hipLaunchKernelGGL(k_gemm_f32, grid, block, 0, st, p, swiglu ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- packing
// Row-major bf16 [N][K] -> fragment order; features past N are zero.
__global__ void k_pack_weight(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int N, int K) {
  const int KS = K >> 5;
  const size_t n16 = (size_t)((N + 15) >> 4) * KS * 64;   // 16-byte lane slots
  for (size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x; q < n16; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q & 63);
    const size_t f = q >> 6;
    const int g = (int)(f / KS), s = (int)(f - (size_t)g * KS);
    const int row = g * 16 + (lane & 15), k = s * 32 + 8 * (lane >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < N) v = *reinterpret_cast<const u32x4*>(src + (size_t)row * K + k);
    *reinterpret_cast<u32x4*>(dst + q * 8) = v;
  }
}

int launch_pack_weight(const void* src, void* dst, int N, int K, hipStream_t st) {
  const size_t n16 = (size_t)((N + 15) >> 4) * (K >> 5) * 64;
  const int blocks = (int)std::min<size_t>((n16 + 255) / 256, 16384);
  hipLaunchKernelGGL(k_pack_weight, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st,
                     reinterpret_cast<const bf16_t*>(src), reinterpret_cast<bf16_t*>(dst), N, K);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Row-major bf16 rows [R][K] -> packed planes: hi = the rows, lo = 0 when xs == 2.
// Also zeroes nzero counters (the sampled head's grid barrier of the same call).
__global__ void k_pack_rows(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int R, int K, size_t plane,
                            int xs, int* zero, int nzero) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  const size_t n = (size_t)R * K;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / K), k = (int)(i - (size_t)r * K);
    const size_t o = frag_off(r, k, K >> 5);
    dst[o] = src[i];
    if (xs == 2) dst[plane + o] = 0;
  }
}

int launch_pack_rows(const void* src, void* dst, int R, int K, size_t plane, int xs, int* zero, int nzero,
                     hipStream_t st) {
  const size_t n = (size_t)R * K;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_pack_rows, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st,
                     reinterpret_cast<const bf16_t*>(src), reinterpret_cast<bf16_t*>(dst), R, K, plane, xs, zero,
                     nzero);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- LM head
// Per row: max logit, sum of exp((z - max) / T), lowest-index argmax, the logit
// of the row's next draft token, and (sampled mode, a lane's last row only)
// the bonus race winner argmax_v z_v / T - ln(-ln U_v).  The logits stay in
// registers; each workgroup (four consecutive 16-token tiles) writes one
// LmPartial per row.

struct RowMeta {
  int next_tok;     // next draft token of the row, -1 on a lane's last row
  int bonus;        // 1 if the row is its lane's last row (bonus draw row)
  uint32_t pos;     // bonus position kv_len + col + 1
  uint32_t lane;
  RowPenalty pen;   // pen.cnt null: no penalties
};

__device__ __forceinline__ RowMeta row_meta(const LmParams& p, int r) {
  RowMeta m;
  const int l = p.ri.row_lane[r], j = p.ri.row_col[r];
  const int last = j == p.ri.lane_cols[l] - 1;
  m.next_tok = last ? -1 : p.tokens[r + 1];
  m.bonus = last;
  m.pos = (uint32_t)(p.kv_len[l] + j + 1);
  m.lane = (uint32_t)l;
  m.pen = row_penalty(p.counts, p.V, p.tokens, p.ri, r, p.presence, p.frequency);
  return m;
}

struct Stat {
  float m, se, zn, gk;
  int arg, gi;
};

__device__ __forceinline__ Stat stat_identity() {
  Stat s;
  s.m = -INFINITY; s.se = 0.f; s.zn = NAN; s.gk = -INFINITY; s.arg = 0x7fffffff; s.gi = 0x7fffffff;
  return s;
}

// Merge b into a (a covers lower token indices than b, or the same range order).
__device__ __forceinline__ Stat stat_merge(Stat a, Stat b, float inv_t) {
  Stat o;
  if (better(b.m, b.arg, a.m, a.arg)) { o.m = b.m; o.arg = b.arg; } else { o.m = a.m; o.arg = a.arg; }
  const float fa = a.m == -INFINITY ? 0.f : expf((a.m - o.m) * inv_t);
  const float fb = b.m == -INFINITY ? 0.f : expf((b.m - o.m) * inv_t);
  o.se = a.se * fa + b.se * fb;
  o.zn = isnan(a.zn) ? b.zn : a.zn;
  if (better(b.gk, b.gi, a.gk, a.gi)) { o.gk = b.gk; o.gi = b.gi; } else { o.gk = a.gk; o.gi = a.gi; }
  return o;
}

// Statistics of four logits z[e] at tokens v0 + e held by one lane (penalties already
// applied), merged across the four lane groups (xor 16, 32) so every lane of a 16-lane
// column ends with the tile's stats.
__device__ __forceinline__ Stat tile_stats(const float (&z)[4], int v0, const RowMeta& rm, const LmParams& p) {
  Stat s;
  float m = z[0]; int a = v0;
#pragma unroll
  for (int e = 1; e < 4; ++e) if (z[e] > m) { m = z[e]; a = v0 + e; }
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    const float om = __shfl_xor(m, x);
    const int oa = __shfl_xor(a, x);
    if (better(om, oa, m, a)) { m = om; a = oa; }
  }
  s.m = m; s.arg = a;
  float se = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) se += expf((z[e] - m) * p.inv_t);
  se += __shfl_xor(se, 16);
  se += __shfl_xor(se, 32);
  s.se = se;
  float zn = -INFINITY;
  if (rm.next_tok >= v0 && rm.next_tok < v0 + 4) zn = z[rm.next_tok - v0];
  zn = fmaxf(zn, __shfl_xor(zn, 16));
  zn = fmaxf(zn, __shfl_xor(zn, 32));
  s.zn = zn == -INFINITY ? NAN : zn;
  float gk = -INFINITY; int gi = 0x7fffffff;
  if (p.sampled && rm.bonus) {
    uint32_t c[4] = {rm.pos, rm.lane, kPurposeRace, (uint32_t)(v0 >> 2)};
    philox4x32_10(c, p.key0, p.key1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float E = -logf(u01(c[e]));
      const float key = z[e] * p.inv_t - logf(E);
      if (better(key, v0 + e, gk, gi)) { gk = key; gi = v0 + e; }
    }
  }
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    const float ok = __shfl_xor(gk, x);
    const int oi = __shfl_xor(gi, x);
    if (better(ok, oi, gk, gi)) { gk = ok; gi = oi; }
  }
  s.gk = gk; s.gi = gi;
  return s;
}

template <int RT, int XS>
__global__ __launch_bounds__(256, 2) void k_lmhead_bf16(LmParams p) {
  constexpr int KC = chunk_steps<RT>(), T = 2;
  using C = CoreShape<RT, T, XS, KC>;
  static_assert(2 * C::NB * 64 * sizeof(u32x4) >= 4 * kMaxRows * sizeof(Stat), "stats fit the X ring");
  __shared__ u32x4 xl[2 * C::NB * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tiles = p.V >> 4, KS = p.H >> 5;
  const bf16_t* W = reinterpret_cast<const bf16_t*>(p.W);
  int tile[T];
  const bf16_t* wp[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    tile[j] = (blockIdx.x * 4 + wave) * T + j;
    wp[j] = W + (size_t)min(tile[j], tiles - 1) * KS * 512 + lane * 8;
  }
  f32x4 acc[T][RT];
#pragma unroll
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  proj_core<RT, T, XS, KC>(wp, 512, reinterpret_cast<const bf16_t*>(p.X), p.xplane, KS, 0, p.H >> 8, xl, acc);
  Stat* sh = reinterpret_cast<Stat*>(xl);   // the core ends on a barrier: the ring is free
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = t * 16 + r16;
    RowMeta rm;
    rm.next_tok = -1; rm.bonus = 0; rm.pos = 0; rm.lane = 0; rm.pen.cnt = nullptr;
    if (r < p.R) rm = row_meta(p, r);
    float pz[T][4] = {};
    if (rm.pen.cnt) {
      int v0[T];
#pragma unroll
      for (int j = 0; j < T; ++j) v0[j] = min(tile[j], tiles - 1) * 16 + 4 * kq;
      penalties4<T>(rm.pen, v0, pz);
    }
    Stat s = stat_identity();
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (tile[j] < tiles) {   // wave-uniform; every lane joins tile_stats' cross-lane shuffles
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = acc[j][t][e] - pz[j][e];
        s = stat_merge(s, tile_stats(z, tile[j] * 16 + 4 * kq, rm, p), p.inv_t);
      }
    }
    if (kq == 0 && r < p.R) sh[wave * kMaxRows + r] = s;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < p.R; r += blockDim.x) {
    Stat s = sh[r];
#pragma unroll
    for (int w = 1; w < 4; ++w) s = stat_merge(s, sh[w * kMaxRows + r], p.inv_t);
    LmPartial o;
    o.m = s.m; o.se = s.se; o.arg = s.arg; o.zn = s.zn; o.gk = s.gk; o.gi = s.gi; o.pad0 = o.pad1 = 0;
    p.part[(size_t)r * p.groups + blockIdx.x] = o;
  }
}

// fp32 weights: one thread per token, one workgroup per 256 tokens of one row.
__global__ void k_lmhead_f32(LmParams p) {
  __shared__ Stat sh[256];
  const int r = blockIdx.y, v = blockIdx.x * 256 + threadIdx.x;
  const float* X = reinterpret_cast<const float*>(p.X) + (size_t)r * p.H;
  const RowMeta rm = row_meta(p, r);
  Stat s = stat_identity();
  if (v < p.V) {
    const float* w = reinterpret_cast<const float*>(p.W) + (size_t)v * p.H;
    double zz = 0.0;
    for (int k = 0; k < p.H; ++k) zz += (double)X[k] * (double)w[k];
    float z = (float)zz;
    if (rm.pen.cnt) z = penalized(z, v, rm.pen);
    s.m = z; s.arg = v; s.se = 1.f;
    s.zn = (rm.next_tok == v) ? z : NAN;
    if (p.sampled && rm.bonus) {
      uint32_t c[4] = {rm.pos, rm.lane, kPurposeRace, (uint32_t)(v >> 2)};
      philox4x32_10(c, p.key0, p.key1);
      const float E = -logf(u01(c[v & 3]));
      s.gk = z * p.inv_t - logf(E);
      s.gi = v;
    }
  }
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] = stat_merge(sh[threadIdx.x], sh[threadIdx.x + w], p.inv_t);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const Stat t = sh[0];
    LmPartial o;
    o.m = t.m; o.se = t.se; o.arg = t.arg; o.zn = t.zn; o.gk = t.gk; o.gi = t.gi; o.pad0 = o.pad1 = 0;
    p.part[(size_t)r * p.groups + blockIdx.x] = o;
  }
}

int launch_lmhead(const LmParams& p, bool bf16, hipStream_t st) {
  if (bf16) {
    const int RT = (p.R + 15) / 16;
    dim3 grid(p.groups), block(256);
#define SV_LM(RT_, XS_) hipLaunchKernelGGL((k_lmhead_bf16<RT_, XS_>), grid, block, 0, st, p)
    if (p.xs == 1) {
      switch (RT) { case 1: SV_LM(1, 1); break; case 2: SV_LM(2, 1); break; case 3: SV_LM(3, 1); break; default: SV_LM(4, 1); }
    } else {
      switch (RT) { case 1: SV_LM(1, 2); break; case 2: SV_LM(2, 2); break; case 3: SV_LM(3, 2); break; default: SV_LM(4, 2); }
    }
#undef SV_LM
  } else {
    dim3 grid(p.groups, p.R), block(256);
    hipLaunchKernelGGL(k_lmhead_f32, grid, block, 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// bf16: one workgroup per 8 token tiles (4 waves x 2 tiles)
int lmhead_groups(int V, bool bf16) { return bf16 ? ((V >> 4) + 7) / 8 : (V + 255) / 256; }

// ------------------------------------------------------------------------------- residual race
// Sampled mode, lanes whose draft i was rejected: the logits of the rejected row (row of
// column i - 1) give p_v = exp((z_v - m) / T) / se, and the exponential race
// argmin_v E_v / max(0, p_v - q_v), E_v = -ln U(seed; position kv_len + i, lane, race, v),
// draws the residual token.  A fallback race with weights p_v is kept alongside for the
// case where every residual weight is 0.  A bf16 model runs it inside the LM head's
// cooperative launch on the logits the workgroups still hold (k_lmhead_coop); an fp32
// model recomputes the row (k_race_f32).

struct RaceKey {
  float k; int i; float fk; int fi;
};

__device__ __forceinline__ bool less_key(float k, int i, float bk, int bi) {
  return k < bk || (k == bk && i < bi);
}

// Penalised logits of the four tokens v0 .. v0 + 3 of row r (raw logits zr).
__device__ __forceinline__ void penalise_row4(float (&z)[4], const float (&zr)[4], int v0, const LmParams& p, int r) {
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = zr[e];
  if (p.counts) {   // the row's penalty, as its statistics had it
    const RowPenalty rp = row_penalty(p.counts, p.V, p.tokens, p.ri, r, p.presence, p.frequency);
    const int vv[1] = {v0};
    float pz[1][4];
    penalties4<1>(rp, vv, pz);
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] -= pz[0][e];
  }
}

// Residual race keys of the four tokens v0 .. v0 + 3 (raw logits zr, the drafter's q at
// the rejected draft's row) for lane l's decision d.
__device__ __forceinline__ void race_lane(const float (&zr)[4], const float (&q)[4], int v0, const LmParams& p, int l,
                                          const LaneDecision& d, RaceKey& rk) {
  float z[4];
  penalise_row4(z, zr, v0, p, d.resid_row);
  const uint32_t pos = (uint32_t)(p.kv_len[l] + d.resid_col);
  uint32_t c[4] = {pos, (uint32_t)l, kPurposeRace, (uint32_t)(v0 >> 2)};
  philox4x32_10(c, p.key0, p.key1);
  // the keys use the hardware exp, log and reciprocal: the winner's margin over the
  // runner-up is of the order of the keys themselves, far above their rounding
  const float rse = __frcp_rn(d.se);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pv = __expf((z[e] - d.m) * p.inv_t) * rse;
    const float w = fmaxf(0.f, pv - q[e]);
    const float E = -__logf(u01(c[e]));
    const float key = w > 0.f ? __fdividef(E, w) : INFINITY;
    const float fkey = pv > 0.f ? __fdividef(E, pv) : INFINITY;
    if (less_key(key, v0 + e, rk.k, rk.i)) { rk.k = key; rk.i = v0 + e; }
    if (less_key(fkey, v0 + e, rk.fk, rk.fi)) { rk.fk = fkey; rk.fi = v0 + e; }
  }
}

// Bonus race keys of lane l (every draft kept) on its last row r: the winner of
// argmax_v z_v / T - ln E_v, E_v = -ln U(seed; position kv_len + k + 1, lane, race, v), kept
// as the minimum of ln E_v - z_v / T (the same values negated, so the same winner).
__device__ __forceinline__ void bonus_lane(const float (&zr)[4], int v0, const LmParams& p, int l, int r,
                                           RaceKey& rk) {
  float z[4];
  penalise_row4(z, zr, v0, p, r);
  const uint32_t pos = (uint32_t)(p.kv_len[l] + p.ri.row_col[r] + 1);
  uint32_t c[4] = {pos, (uint32_t)l, kPurposeRace, (uint32_t)(v0 >> 2)};
  philox4x32_10(c, p.key0, p.key1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float E = -__logf(u01(c[e]));
    const float key = __logf(E) - z[e] * p.inv_t;
    if (less_key(key, v0 + e, rk.k, rk.i)) { rk.k = key; rk.i = v0 + e; }
  }
}

__device__ __forceinline__ RaceKey race_identity() {
  RaceKey r; r.k = INFINITY; r.i = 0x7fffffff; r.fk = INFINITY; r.fi = 0x7fffffff; return r;
}

__device__ __forceinline__ RaceKey race_merge(RaceKey a, RaceKey b) {
  if (less_key(b.k, b.i, a.k, a.i)) { a.k = b.k; a.i = b.i; }
  if (less_key(b.fk, b.fi, a.fk, a.fi)) { a.fk = b.fk; a.fi = b.fi; }
  return a;
}

__device__ __forceinline__ RaceKey race_xor(RaceKey r, int x) {
  RaceKey o;
  o.k = __shfl_xor(r.k, x); o.i = __shfl_xor(r.i, x); o.fk = __shfl_xor(r.fk, x); o.fi = __shfl_xor(r.fi, x);
  return race_merge(r, o);
}

__global__ void k_race_f32(RaceParams p) {
  __shared__ RaceKey sh[256];
  const int l = blockIdx.y, v = blockIdx.x * 256 + threadIdx.x;
  const LaneDecision d = p.dec[l];
  RaceKey rk = race_identity();
  if (d.resid_row >= 0 && v < p.V) {
    const float* X = reinterpret_cast<const float*>(p.X) + (size_t)d.resid_row * p.H;
    const float* w = reinterpret_cast<const float*>(p.W) + (size_t)v * p.H;
    double zz = 0.0;
    for (int k = 0; k < p.H; ++k) zz += (double)X[k] * (double)w[k];
    float z = (float)zz;
    if (p.counts) z = penalized(z, v, row_penalty(p.counts, p.V, p.tokens, p.ri, d.resid_row, p.presence, p.frequency));
    const uint32_t pos = (uint32_t)(p.kv_len[l] + d.resid_col);
    uint32_t c[4] = {pos, (uint32_t)l, kPurposeRace, (uint32_t)(v >> 2)};
    philox4x32_10(c, p.key0, p.key1);
    const float pv = expf((z - d.m) * p.inv_t) / d.se;
    const float wv = fmaxf(0.f, pv - p.q[(size_t)(d.resid_row + 1) * p.V + v]);
    const float E = -logf(u01(c[v & 3]));
    rk.k = wv > 0.f ? E / wv : INFINITY; rk.i = v;
    rk.fk = pv > 0.f ? E / pv : INFINITY; rk.fi = v;
  }
  sh[threadIdx.x] = rk;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] = race_merge(sh[threadIdx.x], sh[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float* o = p.part + ((size_t)l * p.groups + blockIdx.x) * 4;
    o[0] = sh[0].k; o[1] = __int_as_float(sh[0].i); o[2] = sh[0].fk; o[3] = __int_as_float(sh[0].fi);
  }
}

int launch_race(const RaceParams& p, hipStream_t st) {
  dim3 grid(p.groups, p.L), block(256);
  hipLaunchKernelGGL(k_race_f32, grid, block, 0, st, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- sampled LM head
// Sampled rounds of a bf16 model in one cooperative launch, so that no logit is ever
// written to memory ("Draft heads and speculative decoding", "Guess, then check": the
// textbook rule needs the whole row's normaliser before a residual weight is known):
//  1. Workgroup b (one per CU, eight waves) streams the weights of its slice of
//     ceil(V / 16 / G) or one fewer 16-token tiles, in NP passes of 8 T tiles (wave w
//     takes local tiles 8 (q T + j) + w, j < T, in pass q; one pass where the slice fits
//     the accumulators, so the activation is staged once), and keeps every logit of the
//     slice in its accumulators; it writes one statistics partial per row (max,
//     sum exp((z - m) / T), argmax, z at the next draft, the bonus race key), penalties
//     applied.  Greedy rounds stop here (a plain launch; k_row_reduce takes the partials).
//  2. Grid barrier; workgroup r reduces row r's partials in workgroup order.
//  3. Grid barrier; every workgroup reads the row statistics and takes every lane's
//     decision by the textbook rule (the same walk as k_lane_accept), then runs the
//     residual race of each rejecting lane over its own slice, on the logits it still
//     holds, and writes one (key, index) partial per lane; k_accept_coop reduces them.
// Weights are read through a buffer resource spanning the head: a pass slot past the
// workgroup's slice reads out of range (zeros, no memory traffic), so every load sits on
// a straight-line path and the compiler's vmcnt waits stay exact.
constexpr int kCoopWaves = 8;

// Grid barrier of a cooperative launch (every workgroup resident), used once per launch
// with counters that start at zero.  Each thread's agent-coherent stores have completed
// before its workgroup counts itself in, into group b % 8's count (a line of its own); the
// group's last arrival counts the group into the grid's count, which thread 0 of every
// workgroup polls with agent-coherent loads.  Two levels: 256 arrivals on one address
// serialise at the point of coherence (about 9 us a barrier in a probe of 256 workgroups
// against about 4.7 us with groups).  The wait is bounded: past the limit the workgroup
// raises the error flag and goes on, so every wave ends.
__device__ __forceinline__ void grid_barrier(int* cnt, int* groups, int G, int* err, int limit) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x % kCoopGroups;
    const int ng = (G - g + kCoopGroups - 1) / kCoopGroups;   // workgroups of group g
    const int target = G < kCoopGroups ? G : kCoopGroups;     // groups with a workgroup
    if (__hip_atomic_fetch_add(groups + g * 32, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ng - 1)
      __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int spin = 0; __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++spin) {
      if (spin >= limit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Agent-coherent (sc1) 16-byte stores and loads of records whole 16-byte words long,
// element i of the array at `base`: the resource is built on the array (the same for
// every lane), the element offset goes in the lane's VGPR.
template <typename T>
__device__ __forceinline__ void st_coherent16(T* base, uint32_t i, const T& v) {
  static_assert(sizeof(T) % 16 == 0, "16-byte records");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  const u32x4* s = reinterpret_cast<const u32x4*>(&v);
#pragma unroll
  for (int w = 0; w < (int)(sizeof(T) / 16); ++w)
    __builtin_amdgcn_raw_buffer_store_b128(s[w], rs, i * (uint32_t)sizeof(T) + 16 * w, 0, 16);
}
template <typename T>
__device__ __forceinline__ T ld_coherent16(const T* base, uint32_t i) {
  static_assert(sizeof(T) % 16 == 0, "16-byte records");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, 0x7fffffff, 0x00020000);
  T v;
  u32x4* d = reinterpret_cast<u32x4*>(&v);
#pragma unroll
  for (int w = 0; w < (int)(sizeof(T) / 16); ++w)
    d[w] = __builtin_amdgcn_raw_buffer_load_b128(rs, i * (uint32_t)sizeof(T) + 16 * w, 0, 16);
  return v;
}

__device__ __forceinline__ Stat stat_of(const LmPartial& o) {
  Stat s;
  s.m = o.m; s.se = o.se; s.arg = o.arg; s.zn = o.zn; s.gk = o.gk; s.gi = o.gi;
  return s;
}

template <int RT, int XS, int NP, int T>
__global__ __launch_bounds__(512, 1) void k_lmhead_coop(LmParams p) {
  constexpr int NW = kCoopWaves, KC = chunk_steps<RT>(), NC = kUnit / KC;
  constexpr int NB = KC * RT * XS;                 // 1 KB X fragments per chunk
  constexpr int NBW = (NB + NW - 1) / NW;          // staged per wave
  constexpr int RING = 2 * NB * 1024;              // double-buffered X chunk
  constexpr int NLOC = NP * NW * T;                // tile slots of a workgroup
  constexpr int LDSB = RING > 65536 ? RING : 65536;
  constexpr int LB = LDSB / (NLOC * 64) < kMaxLanes ? LDSB / (NLOC * 64) : kMaxLanes;   // race lanes per batch
  static_assert(LB >= 1, "a lane's slice fits LDS");
  static_assert(NW * kMaxRows * sizeof(Stat) <= (size_t)LDSB, "wave stats fit LDS");
  __shared__ __attribute__((aligned(16))) char lds[LDSB];
  __shared__ RowStat srs[kMaxRows];
  __shared__ LaneDecision sdec[kMaxLanes];
  __shared__ int srow[kMaxLanes];   // the row each lane draws from (rejected row, or its last row)
  u32x4* xl = reinterpret_cast<u32x4*>(lds);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int ntiles = p.V >> 4, KS = p.H >> 5, U = p.H >> 8;
  const int G = gridDim.x, b = blockIdx.x;
  const int tb0 = (int)((long long)b * ntiles / G), tb1 = (int)((long long)(b + 1) * ntiles / G);
  const int nloc = tb1 - tb0;
  // row tables (read while the weights stream): the drafter's q of each draft row at its
  // own token, each row's next draft token (-1 on a lane's last row)
  __shared__ float sqd[kMaxRows];
  __shared__ int snext[kMaxRows];
  __shared__ int sslot[kMaxRows];   // race batches: the batch slot of a drawn row, or -1
  if ((int)threadIdx.x < p.R) {
    const int r = threadIdx.x, tk = p.tokens[r];
    const int l = p.ri.row_lane[r], j = p.ri.row_col[r];
    sqd[r] = p.sampled && j > 0 && tk >= 0 && tk < p.V ? p.q[(size_t)r * p.V + tk] : 0.f;
    snext[r] = j == p.ri.lane_cols[l] - 1 ? -1 : p.tokens[r + 1];
  }

  // ---- 1. logits of the slice, pass by pass; X chunks cycle through a double-buffered ring
  const uint32_t wbytes = (uint32_t)((size_t)ntiles * KS * 1024);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.W), 0, (int)wbytes, 0x00020000);
  // slot (pass q, tile j) of wave w holds local tile q NW T + j NW + w
  uint32_t wbase[NP][T];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const int tile = tb0 + (q * T + j) * NW + wave;
      wbase[q][j] = tile < tb1 ? (uint32_t)tile * (uint32_t)KS * 1024u + lane * 16 : wbytes;
    }
  const bf16_t* X = reinterpret_cast<const bf16_t*>(p.X);
  uint32_t xoff[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int bb = min(wave * NBW + i, NB - 1);
    const int pl = bb / (RT * KC), t = (bb / KC) % RT, st = bb % KC;
    xoff[i] = (uint32_t)(pl * p.xplane + ((size_t)t * KS + st) * 512 + lane * 8);
  }
  u32x4 sx[NBW];
  auto stage_load = [&](int stepc) {
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      if (NB % NW == 0 || wave * NBW + i < NB) sx[i] = *reinterpret_cast<const u32x4*>(X + xoff[i] + (size_t)stepc * 512);
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      if (NB % NW == 0 || wave * NBW + i < NB) xl[((size_t)buf * NB + wave * NBW + i) * 64 + lane] = sx[i];
  };
  auto wload = [&](uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 2));   // nt
  };
  f32x4 acc[NP][T][RT];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[q][j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // weight ring: RD steps of the wave's T tiles in flight (a whole unit for up to two
  // tiles, half a unit for up to five, a quarter for more: 16-20 fragments a wave, within
  // the registers of two waves per SIMD)
  constexpr int RD = T > 5 ? kUnit / 4 : T > 2 ? kUnit / 2 : kUnit;
  u32x4 wr[RD][T];
  stage_load(0);
#pragma unroll
  for (int k = 0; k < RD; ++k)
#pragma unroll
    for (int j = 0; j < T; ++j) wr[k][j] = wload(wbase[0][j] + k * 1024);
  stage_store(0);
  __syncthreads();
  int cb = 0;
  const int nchunks = U * NC;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    if (q > 0 && tb0 + q * T * NW >= tb1) break;   // workgroup-uniform: the slice is done
    for (int u = 0; u < U; ++u) {
      // refills RD steps ahead: within this unit, else into unit u + 1 of the pass or unit 0
      // of the next pass
      uint32_t cu[T], nb[T];
#pragma unroll
      for (int j = 0; j < T; ++j) {
        cu[j] = wbase[q][j] + (uint32_t)u * kUnit * 1024u;
        nb[j] = u + 1 < U ? wbase[q][j] + (uint32_t)(u + 1) * kUnit * 1024u : (q + 1 < NP ? wbase[q + 1][j] : wbytes);
      }
#pragma unroll
      for (int h = 0; h < NC; ++h) {
        const int c = u * NC + h;
        stage_load(c + 1 < nchunks ? (c + 1) * KC : 0);   // the next chunk (the X ring cycles over passes)
        // keep the issue order as written: the scheduler would otherwise sink the
        // prefetches next to their first use and expose the full memory latency
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < KC; ++st) {
          const int k = h * KC + st;
          u32x4 xo[XS][RT];
#pragma unroll
          for (int pl = 0; pl < XS; ++pl)
#pragma unroll
            for (int t = 0; t < RT; ++t) xo[pl][t] = xl[((size_t)cb * NB + (pl * RT + t) * KC + st) * 64 + lane];
#pragma unroll
          for (int j = 0; j < T; ++j)
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
              for (int pl = XS - 1; pl >= 0; --pl) acc[q][j][t] = mfma_bf16(wr[k % RD][j], xo[pl][t], acc[q][j][t]);
#pragma unroll
          for (int j = 0; j < T; ++j)
            wr[k % RD][j] = wload(k + RD < kUnit ? cu[j] + (k + RD) * 1024 : nb[j] + (k + RD - kUnit) * 1024);
          __builtin_amdgcn_sched_barrier(0);
        }
        stage_store(cb ^ 1);
        __syncthreads();
        cb ^= 1;
      }
    }
  }

  // ---- per-row statistics of the slice: each lane over its four tokens of every tile of
  // the wave (token order), then across the four lanes of a row, then over the waves in
  // wave order.  The bonus draw is not part of them: it runs after the decisions, for the
  // lanes that keep every draft.
  Stat* sh = reinterpret_cast<Stat*>(lds);   // the ring is free after the last chunk barrier
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = t * 16 + r16;
    const int next_tok = r < p.R ? snext[r] : -1;
    RowPenalty pen;
    pen.cnt = nullptr;
    if (p.counts && r < p.R) pen = row_penalty(p.counts, p.V, p.tokens, p.ri, r, p.presence, p.frequency);
    float z[NP][T][4];
    float m = -INFINITY, zn = -INFINITY;
    int a = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const int tile = tb0 + (q * T + j) * NW + wave;
        const int v0 = tile * 16 + 4 * kq;
        float pz[1][4] = {};
        if (pen.cnt && tile < tb1) {
          const int vv[1] = {v0};
          penalties4<1>(pen, vv, pz);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[q][j][e] = acc[q][j][t][e] - pz[0][e];
          if (tile < tb1) {
            if (z[q][j][e] > m) { m = z[q][j][e]; a = v0 + e; }
            if (v0 + e == next_tok) zn = z[q][j][e];
          }
        }
      }
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float om = __shfl_xor(m, x);
      const int oa = __shfl_xor(a, x);
      if (better(om, oa, m, a)) { m = om; a = oa; }
      zn = fmaxf(zn, __shfl_xor(zn, x));
    }
    float se = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int q = 0; q < NP; ++q)
#pragma unroll
        for (int j = 0; j < T; ++j)
          if (tb0 + (q * T + j) * NW + wave < tb1)
#pragma unroll
            for (int e = 0; e < 4; ++e) se += __expf((z[q][j][e] - m) * p.inv_t);
    }
    se += __shfl_xor(se, 16);
    se += __shfl_xor(se, 32);
    if (kq == 0 && r < p.R) {
      Stat s;
      s.m = m; s.arg = a; s.se = se; s.zn = zn == -INFINITY ? NAN : zn; s.gk = -INFINITY; s.gi = 0x7fffffff;
      sh[wave * kMaxRows + r] = s;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < p.R) {
    const int r = threadIdx.x;
    Stat s = sh[r];
#pragma unroll
    for (int w = 1; w < NW; ++w) s = stat_merge(s, sh[w * kMaxRows + r], p.inv_t);
    LmPartial o;
    o.m = s.m; o.se = s.se; o.arg = s.arg; o.zn = s.zn; o.gk = s.gk; o.gi = s.gi; o.pad0 = o.pad1 = 0;
    if (p.sampled) st_coherent16(p.part, (uint32_t)(b * p.R + r), o);
    else p.part[(size_t)r * G + b] = o;   // greedy: row-major partials for k_row_reduce, nothing else
  }
  if (!p.sampled) return;
  if (b == 0 && threadIdx.x == 0) __hip_atomic_store(p.bar + 3, G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  grid_barrier(p.bar + 0, p.bar + kCoopGroupBase, G, p.bar + 2, p.spin_limit);

  // ---- 2. row r's partials in workgroup order: 256 threads, a fixed tree
  for (int r = b; r < p.R; r += G) {   // workgroup-uniform
    float* fm = reinterpret_cast<float*>(lds);
    float* fse = fm + 256;
    float* fzn = fm + 512;
    float* fgk = fm + 768;
    int* iarg = reinterpret_cast<int*>(fm + 1024);
    int* igi = iarg + 256;
    const int t = threadIdx.x;
    if (t < 256) {
      Stat s = stat_identity();
      for (int g = (int)((long long)t * G / 256); g < (int)((long long)(t + 1) * G / 256); ++g)
        s = stat_merge(s, stat_of(ld_coherent16(p.part, (uint32_t)(g * p.R + r))), p.inv_t);
      fm[t] = s.m; fse[t] = s.se; fzn[t] = s.zn; fgk[t] = s.gk; iarg[t] = s.arg; igi[t] = s.gi;
    }
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (t < w) {
        Stat a, c;
        a.m = fm[t]; a.se = fse[t]; a.zn = fzn[t]; a.gk = fgk[t]; a.arg = iarg[t]; a.gi = igi[t];
        c.m = fm[t + w]; c.se = fse[t + w]; c.zn = fzn[t + w]; c.gk = fgk[t + w]; c.arg = iarg[t + w]; c.gi = igi[t + w];
        a = stat_merge(a, c, p.inv_t);
        fm[t] = a.m; fse[t] = a.se; fzn[t] = a.zn; fgk[t] = a.gk; iarg[t] = a.arg; igi[t] = a.gi;
      }
      __syncthreads();
    }
    if (t == 0) {
      RowStat o;
      o.m = fm[0]; o.se = fse[0]; o.zn = fzn[0]; o.gk = fgk[0]; o.arg = iarg[0]; o.gi = igi[0]; o.pad0 = o.pad1 = 0;
      st_coherent16(p.rstat, (uint32_t)r, o);
    }
    __syncthreads();
  }
  grid_barrier(p.bar + 1, p.bar + kCoopGroupBase + kCoopGroups * 32, G, p.bar + 2, p.spin_limit);

  // ---- 3. every lane's decision, then each lane's draw over the slice: the residual race of
  // a lane that rejected a draft, the bonus race (Gumbel-max on z / T, as a minimum of
  // ln E_v - z_v / T) of a lane that kept them all
  if ((int)threadIdx.x < p.R) {
    const int r = threadIdx.x;
    srs[r] = ld_coherent16(p.rstat, (uint32_t)r);
  }
  __syncthreads();
  if ((int)threadIdx.x < p.ri.L) {
    const int l = threadIdx.x;
    auto qd = [&](int r) { return sqd[r]; };
    const LaneDecision d = decide_sampled(srs, p.tokens, p.kv_len, qd, p.inv_t, p.key0, p.key1, p.ri, l, nullptr);
    sdec[l] = d;
    srow[l] = d.resid_row >= 0 ? d.resid_row : p.ri.lane_start[l + 1] - 1;
    if (b == 0) p.dec[l] = d;
  }
  __syncthreads();
  const int L = p.ri.L;
  float* zl = reinterpret_cast<float*>(lds);   // [LB][NLOC][16] logits of the drawn rows
  constexpr int GI = (NLOC * 4 + 63) / 64;     // four-token groups per lane of a wave
  for (int b0 = 0; b0 < L; b0 += LB) {
    const int nb = min(LB, L - b0);
    __syncthreads();   // the previous batch has read zl and sslot
    if ((int)threadIdx.x < kMaxRows) sslot[threadIdx.x] = -1;
    __syncthreads();
    if ((int)threadIdx.x < nb) sslot[srow[b0 + threadIdx.x]] = threadIdx.x;
    __syncthreads();
    // each lane writes the drawn rows among its own (rows 16 t + r16)
    int slot[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) slot[t] = sslot[t * 16 + r16];
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const int lt = (q * T + j) * NW + wave;
        if (tb0 + lt < tb1) {
#pragma unroll
          for (int t = 0; t < RT; ++t)
            if (slot[t] >= 0) *reinterpret_cast<f32x4*>(zl + ((size_t)slot[t] * NLOC + lt) * 16 + 4 * kq) = acc[q][j][t];
        }
      }
    __syncthreads();
    for (int i = wave; i < nb; i += NW) {   // wave-uniform
      const int l = b0 + i;
      const LaneDecision d = sdec[l];
      const bool resid = d.resid_row >= 0;
      const int rr = srow[l];
      RaceKey rk = race_identity();
      // every group's logits and q first, then the keys
      f32x4 zv[GI], qv[GI];
#pragma unroll
      for (int gi = 0; gi < GI; ++gi) {
        const int g = min(gi * 64 + lane, max(nloc * 4 - 1, 0));
        const int lt = g >> 2, v0 = (tb0 + lt) * 16 + 4 * (g & 3);
        zv[gi] = *reinterpret_cast<const f32x4*>(zl + ((size_t)i * NLOC + lt) * 16 + 4 * (g & 3));
        qv[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (resid && nloc > 0) qv[gi] = *reinterpret_cast<const f32x4*>(p.q + (size_t)(rr + 1) * p.V + v0);
      }
#pragma unroll
      for (int gi = 0; gi < GI; ++gi) {
        const int g = gi * 64 + lane;
        if (g < nloc * 4) {
          const int v0 = (tb0 + (g >> 2)) * 16 + 4 * (g & 3);
          const float z[4] = {zv[gi][0], zv[gi][1], zv[gi][2], zv[gi][3]};
          const float qq[4] = {qv[gi][0], qv[gi][1], qv[gi][2], qv[gi][3]};
          if (resid) race_lane(z, qq, v0, p, l, d, rk);
          else bonus_lane(z, v0, p, l, rr, rk);
        }
      }
#pragma unroll
      for (int x = 1; x <= 32; x <<= 1) rk = race_xor(rk, x);
      if (lane == 0) {
        float* o = p.racep + ((size_t)l * G + b) * 4;
        o[0] = rk.k; o[1] = __int_as_float(rk.i); o[2] = rk.fk; o[3] = __int_as_float(rk.fi);
      }
    }
  }
}

// Workgroups of the cooperative head: one per CU of the current device, at most kCUs.
int coop_grid() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  const int g = std::min(cus, kCUs);
  if (dev < 64) cached[dev] = g;
  return g;
}

// Slice shape of the cooperative head: T tiles per wave and pass, NP passes of 8 T tiles,
// rounded up to an instantiated count.  One pass of five tiles per wave (eight with at
// most two row tiles) stages the activation once; smaller slices take passes of two tiles
// per wave (16 KB of weights in flight per wave); one tile per wave in up to eight passes
// where four passes of two would hold more accumulators than the registers of two waves
// per SIMD.
struct CoopShape {
  int np, t;
};

static CoopShape coop_shape(int V, int grid, int RT) {
  const int per = (V / 16 + grid - 1) / grid;
  // one pass of up to five tiles per wave (eight with at most two row tiles): the
  // activation is staged once
  const int t1 = (per + kCoopWaves - 1) / kCoopWaves;
  if (t1 > 2 && t1 <= 5) return CoopShape{1, 5};
  if (t1 > 5 && t1 <= 8 && RT <= 2) return CoopShape{1, 8};
  const int np2 = (per + 2 * kCoopWaves - 1) / (2 * kCoopWaves);
  if (np2 <= 3 || (np2 == 4 && RT <= 2)) return CoopShape{std::max(np2, 1), 2};
  const int np1 = (per + kCoopWaves - 1) / kCoopWaves;
  if (np1 <= 8) return CoopShape{8, 1};
  return CoopShape{0, 0};
}

int launch_lmhead_coop(const LmParams& p0, int grid, hipStream_t st) {
  LmParams p = p0;
  if (grid < 1) return -1;
  const int RT = (p.R + 15) / 16;
  const CoopShape cs = coop_shape(p.V, grid, RT);
  if (cs.np == 0 || (size_t)p.V * p.H * 2 > 0x80000000ull) return -2;
  p.groups = grid;
  const void* f = nullptr;
#define SV_C(RT_, XS_, NP_, T_) f = reinterpret_cast<const void*>(&k_lmhead_coop<RT_, XS_, NP_, T_>)
#define SV_C_NP(RT_, XS_)                                    \
  if (cs.t == 1) {                                           \
    if constexpr (RT_ >= 3) SV_C(RT_, XS_, 8, 1);            \
  } else if (cs.t == 5) {                                    \
    SV_C(RT_, XS_, 1, 5);                                    \
  } else if (cs.t == 8) {                                    \
    if constexpr (RT_ <= 2) SV_C(RT_, XS_, 1, 8);            \
  } else {                                                   \
    switch (cs.np) {                                         \
      case 1: SV_C(RT_, XS_, 1, 2); break;                   \
      case 2: SV_C(RT_, XS_, 2, 2); break;                   \
      case 3: SV_C(RT_, XS_, 3, 2); break;                   \
      default: if constexpr (RT_ <= 2) SV_C(RT_, XS_, 4, 2); break; \
    }                                                        \
  }
#define SV_C_RT(XS_)                  \
  switch (RT) {                       \
    case 1: SV_C_NP(1, XS_); break;   \
    case 2: SV_C_NP(2, XS_); break;   \
    case 3: SV_C_NP(3, XS_); break;   \
    default: SV_C_NP(4, XS_); break;  \
  }
  if (p.xs == 1) {
    SV_C_RT(1);
  } else {
    SV_C_RT(2);
  }
#undef SV_C_RT
#undef SV_C_NP
#undef SV_C
  if (!f) return -2;
  void* args[] = {&p};
  // greedy statistics need no grid barrier: a plain launch of the same one-per-CU grid
  const hipError_t e = p.sampled ? hipLaunchCooperativeKernel(f, dim3(grid), dim3(kCoopWaves * 64), args, 0, st)
                                 : hipLaunchKernel(f, dim3(grid), dim3(kCoopWaves * 64), args, 0, st);
  return e == hipSuccess ? 0 : -1;
}

}  // namespace sv
