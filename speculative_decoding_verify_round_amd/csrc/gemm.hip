// Skinny-M projections and the fused LM head of the verify round (gfx950).
//
// A verify round multiplies at most 64 rows by every weight matrix of the
// model; the pass is bound by streaming the weights from HBM once ("that pass
// is mostly the card streaming the weights from memory", "Speculative
// decoding", gpillon.github.io/ignis).  Each wave owns 16 output features
// (16 rows of W, one or two matrices) over a contiguous range of 256-wide K
// chunks and multiplies them against all rows of X with
// v_mfma_f32_16x16x32_bf16: W is the A operand (16 features), X the B operand
// (16 rows per tile, up to four tiles).  Weights are loaded with non-temporal
// 16-byte loads into an eight-step register ring, so eight MFMA steps of W
// (and of X, issued at the same distance so the in-order vmcnt counter never
// makes a step wait on a younger load) are in flight per wave.
//
// The K split of a matrix is a function of its shape only, and every output
// element is one MFMA accumulation chain in a fixed K order, so a row's result
// never depends on how many rows the round carries.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

constexpr int kSteps = 8;   // MFMA k-steps (32 each) per 256-wide chunk
constexpr int kRingW = 8;   // k-steps of W in flight per wave
constexpr int kRingX = 2;   // k-steps of X in flight per wave (L1/L2 hits)

// acc[m][t][e] += W_m[16 features][k] . X[16 rows of tile t][k] over k-chunks [c0, c1).
// X arrives as XS bf16 planes (hi, lo); each k-step chains the planes' MFMAs
// (lo first) from a zero accumulator, and the step's fp32 result is added to a
// float64 accumulator, so the K sum carries about one fp32 ulp of error.
// Loads are issued X(step + 2) before W(step + 8) so that waiting for an X
// step never waits for the younger W loads behind it (vmcnt counts in order).
template <int RT, int NMAT, int XS>
__device__ __forceinline__ void gemm_core(const bf16_t* const (&wb)[NMAT], const bf16_t* const (&xb)[XS][RT],
                                          int c0, int c1, double (&acc)[NMAT][RT][4]) {
  if (c0 >= c1) return;
  const int s0 = c0 * kSteps, ns = (c1 - c0) * kSteps;   // a multiple of kRingW
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  u32x4 wr[kRingW][NMAT];
  u32x4 xr[kRingX][XS][RT];
  auto loadW = [&](int slot, int st) {
    const int k = (s0 + st) * 32;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wr[slot][m] = ld_stream(reinterpret_cast<const u32x4*>(wb[m] + k));
  };
  auto loadX = [&](int slot, int st) {
    const int k = (s0 + st) * 32;
#pragma unroll
    for (int x = 0; x < XS; ++x)
#pragma unroll
      for (int t = 0; t < RT; ++t) xr[slot][x][t] = *reinterpret_cast<const u32x4*>(xb[x][t] + k);
  };
  auto step = [&](int ws, int xsl) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        f32x4 d = zero;
#pragma unroll
        for (int x = XS - 1; x >= 0; --x) d = mfma_bf16(wr[ws][m], xr[xsl][x][t], d);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[m][t][e] += (double)d[e];
      }
  };
#pragma unroll
  for (int u = 0; u < kRingX; ++u) loadX(u, u);
#pragma unroll
  for (int u = 0; u < kRingW; ++u) loadW(u, u);
  for (int i = 0; i < ns - kRingW; i += kRingW) {
#pragma unroll
    for (int u = 0; u < kRingW; ++u) {
      step(u, u % kRingX);
      loadX(u % kRingX, i + u + kRingX);
      loadW(u, i + u + kRingW);
    }
  }
#pragma unroll
  for (int u = 0; u < kRingW; ++u) {
    step(u, u % kRingX);
    if (u + kRingX < kRingW) loadX(u % kRingX, ns - kRingW + u + kRingX);
  }
}

// float(silu(g) * u) evaluated in float64 from the fp32-rounded projections
__device__ __forceinline__ float swiglu(double g64, double u64) {
  const double g = (double)(float)g64, u = (double)(float)u64;
  return (float)(g / (1.0 + exp(-g)) * u);
}

// ------------------------------------------------------------------------------- projection
template <int RT, int NMAT, bool SWIGLU, int XS>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  if (gw >= p.groups * p.S) return;
  const int g = gw % p.groups, s = gw / p.groups;
  const int C = p.K >> 8;
  const int c0 = (int)((long long)s * C / p.S), c1 = (int)((long long)(s + 1) * C / p.S);
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = g * 16;
  const int nrow = min(n0 + r16, p.N - 1);   // features past N read a valid row; never stored
  const bf16_t* wb[NMAT];
  wb[0] = p.W0 + (size_t)nrow * p.K + kq * 8;
  if constexpr (NMAT > 1) wb[1] = p.W1 + (size_t)nrow * p.K + kq * 8;
  const bf16_t* xb[XS][RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const size_t off = (size_t)min(t * 16 + r16, p.R - 1) * p.K + kq * 8;
    xb[0][t] = p.Xh + off;
    if constexpr (XS > 1) xb[1][t] = p.Xl + off;
  }
  double acc[NMAT][RT][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[m][t][e] = 0.0;
  gemm_core<RT, NMAT, XS>(wb, xb, c0, c1, acc);
  // lane holds D[feature n0 + 4 kq + e][row t * 16 + r16]
  const size_t plane = (size_t)p.R * p.N;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = t * 16 + r16;
    if (r >= p.R) continue;
    const int nf = n0 + 4 * kq;
    if constexpr (!SWIGLU) {
      if (nf + 4 <= p.N) {
        *reinterpret_cast<f32x4*>(p.P + ((size_t)s * p.R + r) * p.N + nf) =
            f32x4{(float)acc[0][t][0], (float)acc[0][t][1], (float)acc[0][t][2], (float)acc[0][t][3]};
      } else {
        for (int e = 0; e < 4 && nf + e < p.N; ++e) p.P[((size_t)s * p.R + r) * p.N + nf + e] = (float)acc[0][t][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nf + e < p.N) st_planes(p.Yb + (size_t)r * p.N + nf + e, plane, swiglu(acc[0][t][e], acc[1][t][e]));
    }
  }
}

int launch_gemm_bf16(const GemmParams& p, int nmat, bool swiglu, hipStream_t st) {
  const int RT = (p.R + 15) / 16;
  const int waves = p.groups * p.S;
  const bool two = p.Xl != nullptr;
  dim3 grid((waves + 3) / 4), block(256);
#define SV_GEMM(RT_, NM_, SW_, XS_) hipLaunchKernelGGL((k_gemm_bf16<RT_, NM_, SW_, XS_>), grid, block, 0, st, p)
#define SV_GEMM_RT(NM_, SW_, XS_)             \
  switch (RT) {                               \
    case 1: SV_GEMM(1, NM_, SW_, XS_); break; \
    case 2: SV_GEMM(2, NM_, SW_, XS_); break; \
    case 3: SV_GEMM(3, NM_, SW_, XS_); break; \
    default: SV_GEMM(4, NM_, SW_, XS_); break; \
  }
  if (nmat == 1) {
    if (two) { SV_GEMM_RT(1, false, 2); } else { SV_GEMM_RT(1, false, 1); }
  } else {
    SV_GEMM_RT(2, true, 2);   // two matrices only ever feed the SwiGLU epilogue
  }
  (void)swiglu;
#undef SV_GEMM_RT
#undef SV_GEMM
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
    p.Ya[(size_t)r * p.N + n] = swiglu(a, b);
  }
}

int launch_gemm_f32(const GemmF32Params& p, bool swiglu, hipStream_t st) {
  dim3 grid((p.N + 255) / 256, p.R), block(256);
  hipLaunchKernelGGL(k_gemm_f32, grid, block, 0, st, p, swiglu ? 1 : 0);
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
};

__device__ __forceinline__ RowMeta row_meta(const LmParams& p, int r) {
  RowMeta m;
  const int l = p.ri.row_lane[r], j = p.ri.row_col[r];
  const int last = j == p.ri.lane_cols[l] - 1;
  m.next_tok = last ? -1 : p.tokens[r + 1];
  m.bonus = last;
  m.pos = (uint32_t)(p.kv_len[l] + j + 1);
  m.lane = (uint32_t)l;
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

// Statistics of four logits z[e] at tokens v0 + e held by one lane, merged across the
// four lane groups (xor 16, 32) so every lane of a 16-lane column ends with the tile's stats.
__device__ __forceinline__ Stat tile_stats(const float z[4], int v0, const RowMeta& rm, const LmParams& p) {
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
  __shared__ Stat sh[4][kMaxRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tiles = p.V >> 4;
  const int tile = blockIdx.x * 4 + wave;
  const bool valid = tile < tiles;
  double acc[1][RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[0][t][e] = 0.0;
  if (valid) {
    const bf16_t* X = reinterpret_cast<const bf16_t*>(p.X);
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.W);
    const bf16_t* wb[1] = {W + (size_t)(tile * 16 + r16) * p.H + kq * 8};
    const bf16_t* xb[XS][RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const size_t off = (size_t)min(t * 16 + r16, p.R - 1) * p.H + kq * 8;
      xb[0][t] = X + off;
      if constexpr (XS > 1) xb[1][t] = X + (size_t)p.R * p.H + off;
    }
    gemm_core<RT, 1, XS>(wb, xb, 0, p.H >> 8, acc);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = t * 16 + r16;
    Stat s = stat_identity();
    if (valid) {   // wave-uniform; every lane joins tile_stats' cross-lane shuffles
      RowMeta rm;
      rm.next_tok = -1; rm.bonus = 0; rm.pos = 0; rm.lane = 0;
      if (r < p.R) rm = row_meta(p, r);
      const float z[4] = {(float)acc[0][t][0], (float)acc[0][t][1], (float)acc[0][t][2], (float)acc[0][t][3]};
      s = tile_stats(z, tile * 16 + 4 * kq, rm, p);
      if (r >= p.R) s = stat_identity();
    }
    if (kq == 0 && r < p.R) sh[wave][r] = s;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < p.R; r += blockDim.x) {
    Stat s = sh[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) s = stat_merge(s, sh[w][r], p.inv_t);
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
    const float z = (float)zz;
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

int lmhead_groups(int V, bool bf16) { return bf16 ? ((V >> 4) + 3) / 4 : (V + 255) / 256; }

// ------------------------------------------------------------------------------- residual race
// Sampled mode, lanes whose draft i was rejected: recompute the logits of the
// rejected row (row of column i - 1), form p_v = exp((z_v - m) / T) / se, and
// run the exponential race argmin_v E_v / max(0, p_v - q_v) with
// E_v = -ln U(seed; position kv_len + i, lane, race, v).  A fallback race with
// weights p_v is kept alongside for the case where every residual weight is 0.

struct RaceKey {
  float k; int i; float fk; int fi;
};

__device__ __forceinline__ bool less_key(float k, int i, float bk, int bi) {
  return k < bk || (k == bk && i < bi);
}

__device__ __forceinline__ void race_lane(const float z[4], int v0, const RaceParams& p, int l, RaceKey& rk) {
  const LaneDecision d = p.dec[l];
  const int qrow = d.resid_row + 1;
  const uint32_t pos = (uint32_t)(p.kv_len[l] + d.resid_col);
  uint32_t c[4] = {pos, (uint32_t)l, kPurposeRace, (uint32_t)(v0 >> 2)};
  philox4x32_10(c, p.key0, p.key1);
  const float* q = p.q + (size_t)qrow * p.V + v0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pv = expf((z[e] - d.m) * p.inv_t) / d.se;
    const float w = fmaxf(0.f, pv - q[e]);
    const float E = -logf(u01(c[e]));
    const float key = w > 0.f ? E / w : INFINITY;
    const float fkey = pv > 0.f ? E / pv : INFINITY;
    if (less_key(key, v0 + e, rk.k, rk.i)) { rk.k = key; rk.i = v0 + e; }
    if (less_key(fkey, v0 + e, rk.fk, rk.fi)) { rk.fk = fkey; rk.fi = v0 + e; }
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

template <int RT, int XS>
__global__ __launch_bounds__(256, 2) void k_race_bf16(RaceParams p) {
  __shared__ RaceKey sh[4][kMaxLanes];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tiles = p.V >> 4;
  const int tile = blockIdx.x * 4 + wave;
  const bool valid = tile < tiles;
  // any lane with a rejection?  (uniform across the workgroup)
  bool any = false;
  for (int l = 0; l < p.L; ++l) any |= p.dec[l].resid_row >= 0;
  if (!any) return;
  double acc[1][RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[0][t][e] = 0.0;
  if (valid) {
    const bf16_t* X = reinterpret_cast<const bf16_t*>(p.X);
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.W);
    const bf16_t* wb[1] = {W + (size_t)(tile * 16 + r16) * p.H + kq * 8};
    const bf16_t* xb[XS][RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int l = min(t * 16 + r16, p.L - 1);
      const int row = max(p.dec[l].resid_row, 0);
      xb[0][t] = X + (size_t)row * p.H + kq * 8;
      if constexpr (XS > 1) xb[1][t] = X + (size_t)p.R * p.H + (size_t)row * p.H + kq * 8;
    }
    gemm_core<RT, 1, XS>(wb, xb, 0, p.H >> 8, acc);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int l = t * 16 + r16;
    RaceKey rk = race_identity();
    if (valid && l < p.L && p.dec[l].resid_row >= 0) {
      const float z[4] = {(float)acc[0][t][0], (float)acc[0][t][1], (float)acc[0][t][2], (float)acc[0][t][3]};
      race_lane(z, tile * 16 + 4 * kq, p, l, rk);
    }
    rk = race_xor(rk, 16);
    rk = race_xor(rk, 32);
    if (kq == 0 && l < p.L) sh[wave][l] = rk;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < p.L; l += blockDim.x) {
    RaceKey r = sh[0][l];
    for (int w = 1; w < 4; ++w) r = race_merge(r, sh[w][l]);
    float* o = p.part + ((size_t)l * p.groups + blockIdx.x) * 4;
    o[0] = r.k; o[1] = __int_as_float(r.i); o[2] = r.fk; o[3] = __int_as_float(r.fi);
  }
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
    const float z = (float)zz;
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

int launch_race(const RaceParams& p, bool bf16, hipStream_t st) {
  if (bf16) {
    const int RT = (p.L + 15) / 16;
    dim3 grid(p.groups), block(256);
#define SV_RACE(RT_, XS_) hipLaunchKernelGGL((k_race_bf16<RT_, XS_>), grid, block, 0, st, p)
    if (p.xs == 1) {
      switch (RT) { case 1: SV_RACE(1, 1); break; case 2: SV_RACE(2, 1); break; case 3: SV_RACE(3, 1); break; default: SV_RACE(4, 1); }
    } else {
      switch (RT) { case 1: SV_RACE(1, 2); break; case 2: SV_RACE(2, 2); break; case 3: SV_RACE(3, 2); break; default: SV_RACE(4, 2); }
    }
#undef SV_RACE
  } else {
    dim3 grid(p.groups, p.L), block(256);
    hipLaunchKernelGGL(k_race_f32, grid, block, 0, st, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
