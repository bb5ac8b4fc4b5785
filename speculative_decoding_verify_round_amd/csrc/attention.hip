// Verify attention (gfx950).
//
// "Speculative decoding" (gpillon.github.io/ignis), "One round, step by step",
// step 3: all of a lane's columns (anchor plus drafts) go through the layer in
// one pass; column j attends to the lane's committed cache and to its own
// columns 0..j (causal among the columns of the round).
//
// One workgroup handles (lane, kv head, chunk of `chunk` absolute positions);
// its four waves take consecutive quarters of the chunk.  All (k+1) x G query
// rows of the lane/kv-head pair are processed together, so every K/V byte of
// the lane is read once per layer.  Positions are tiled by absolute position:
// a 16-position tile may hold committed keys (paged cache) and this round's
// own columns (staged in the workspace) side by side, and the online softmax
// visits tiles, waves and chunks in positional order.  A row's result is
// therefore independent of how many columns the round carries and of whether
// a key is still staged or already committed.
//
// bf16 path (head_dim 128): the workgroup stages 64-position K and V tiles in
// LDS (the next tile's loads are in flight while the current one is used);
// wave w owns query tile w (16 of the lane's (k+1) x G query rows) over the
// whole chunk.  Per 32 positions:
//   S^T[pos][query] = K . Q^T with v_mfma_f32_16x16x32_bf16 (K rows = A; the
//   float32 queries = B, as bf16 hi + lo planes);
//   P = exp2(S * log2(e)/sqrt(d) - m) in fp32, split into bf16 hi + lo;
//   O^T[d][query] += V^T . P^T.  The V pool is stored d-major inside a block
//   ([d][16 slots]) so that V^T tiles are contiguous; the lane's key order
//   inside the K = 32 MFMA step equals the order in which the S^T result left
//   it, so P needs no shuffle.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace sv {

template <int QT>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnParams p) {
  constexpr int D = 128, STEP = 64, KP = D + 8, VP = STEP + 8, PW = kAttnPartPad + D;
  __shared__ bf16_t Ks[STEP * KP];   // [position][d], rows padded by 16 B
  __shared__ bf16_t Vs[D * VP];      // [d][position], rows padded by 16 B
  __shared__ int sblk[kMaxChunk / kBlock];   // the chunk's block ids
  const int c = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int pos0 = c * p.chunk;
  if (pos0 >= end) return;
  const int Mq = cols * p.G;
  const int cend = min(pos0 + p.chunk, end);
  const int nsteps = (cend - pos0 + STEP - 1) / STEP;
  const int* bt = p.block_table + (size_t)l * p.max_blocks;
  // block ids of the chunk, looked up once (a table entry past the lane's blocks is never used)
  for (int i = tid; i < p.chunk / kBlock; i += blockDim.x) {
    const int b = pos0 / kBlock + i;
    sblk[i] = b < p.max_blocks ? clamp_blk(bt[b], p.n_blocks) : 0;
  }
  __syncthreads();
  const float* Qp = p.q;
  const bf16_t* Kp = reinterpret_cast<const bf16_t*>(p.kpool);
  const bf16_t* Vp = reinterpret_cast<const bf16_t*>(p.vpool);
  const bf16_t* SK = reinterpret_cast<const bf16_t*>(p.sk);
  const bf16_t* SV = reinterpret_cast<const bf16_t*>(p.sv);
  const int nkv = p.nkv;

  // ---- cooperative staging of one 64-position step: 4 K items and 4 V items of 16 B per thread
  u32x4 kreg[1][4], vreg[1][4];
  // Every load is issued unconditionally from a valid address (a position past the
  // lane's live range reads a clamped one and is zeroed), so the loads carry no
  // divergent branches; only the block that straddles the cached/staged boundary
  // takes the (workgroup-uniform) element-wise V path.
  auto load_step = [&](int s, auto set_tag) {
    constexpr int B = decltype(set_tag)::value;
    const int base = pos0 + s * STEP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = base + (tid >> 4) + 16 * j, seg = tid & 15;
      const int srow = min(max(pos - kvl, 0), cols - 1);
      const bf16_t* kc = Kp + (((size_t)sblk[(pos - pos0) >> 4] * nkv + g) * kBlock + (pos & 15)) * D;
      const bf16_t* ks = SK + ((size_t)(rs + srow) * nkv + g) * D;
      const u32x4 v = *reinterpret_cast<const u32x4*>((pos < kvl ? kc : ks) + seg * 8);
      kreg[B][j] = pos < end ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bpos = base + 16 * j, d = tid >> 1, hf = tid & 1;
      const int blk = sblk[(bpos - pos0) >> 4];
      const bf16_t* vb = Vp + (((size_t)blk * nkv + g) * D + d) * kBlock;
      if (bpos + 16 <= kvl) {
        vreg[B][j] = *reinterpret_cast<const u32x4*>(vb + hf * 8);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t two = 0;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int pos = bpos + hf * 8 + 2 * e2 + hh;
            const int srow = min(max(pos - kvl, 0), cols - 1);
            const bf16_t vc = vb[pos & 15];
            const bf16_t vs = SV[((size_t)(rs + srow) * nkv + g) * D + d];
            const bf16_t v = pos < kvl ? vc : (pos < end ? vs : (bf16_t)0);
            two |= (uint32_t)v << (16 * hh);
          }
          w[e2] = two;
        }
        vreg[B][j] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  auto store_step = [&](auto set_tag) {
    constexpr int B = decltype(set_tag)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(Ks + ((tid >> 4) + 16 * j) * KP + (tid & 15) * 8) = kreg[B][j];
      *reinterpret_cast<u32x4*>(Vs + (tid >> 1) * VP + 16 * j + (tid & 1) * 8) = vreg[B][j];
    }
  };

  // ---- this wave's query tile: rows m = wave*16 + r16 (column j = m / G, head g*G + m % G)
  const bool owner = wave < QT && wave * 16 < Mq;
  const int m = wave * 16 + r16;
  u32x4 qh[4], ql[4];            // the float32 query as bf16 hi + lo planes
  int lim = -1;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) { qh[ds] = u32x4{0u, 0u, 0u, 0u}; ql[ds] = qh[ds]; }
  if (owner && m < Mq) {
    const int j = m / p.G, hh = m - j * p.G;
    const float* ptr = Qp + ((size_t)(rs + j) * p.nq + g * p.G + hh) * D + kq * 8;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(ptr + ds * 32);
      const f32x4 b = *reinterpret_cast<const f32x4*>(ptr + ds * 32 + 4);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t hw, lw;
        split2(v[2 * i], v[2 * i + 1], hw, lw);
        qh[ds][i] = hw;
        ql[ds][i] = lw;
      }
    }
    lim = kvl + j;
  }
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 64-position step: S^T for the four 16-position tiles, one online-softmax
  // update (max, rescale, exp) for all 64 positions, then O^T += V^T P^T over
  // two 32-position MFMA steps.
  auto compute_step = [&](int s) {
    const int p0 = pos0 + s * STEP;
    f32x4 sc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16_t* kr = Ks + (st * 16 + r16) * KP + kq * 8;
      sc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kr + ds * 32);
        sc[st] = mfma_bf16(kf, ql[ds], sc[st]);
        sc[st] = mfma_bf16(kf, qh[ds], sc[st]);
      }
    }
    // lane holds S^T[p0 + 16 st + 4 kq + e][query m]
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = p0 + st * 16 + 4 * kq + e;
        const float v = pos <= lim ? sc[st][e] * p.scale_log2 : -INFINITY;
        x[st * 4 + e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    float pr[16];
    float alpha = 1.f;
    if (mnew == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = 0.f;
    } else {
      // arguments are <= 0: the raw v_exp_f32 (results below 2^-126 flush to 0)
      alpha = __builtin_amdgcn_exp2f(mrun - mnew);
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ps += pr[i];
    lrun = lrun * alpha + ps;
    mrun = mnew;
    // P = hi + lo in bf16 (what is left is below 2^-17 P); MFMA step c covers tiles 2c and 2c + 1
    u32x4 ph[2], pl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t hw, lw;
        split2(pr[8 * c + 2 * i], pr[8 * c + 2 * i + 1], hw, lw);
        ph[c][i] = hw;
        pl[c][i] = lw;
      }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
    // O^T[d][m] += V^T[d][keys] P^T[keys][m]; the lane's keys are (tile 2c + h, 4 kq .. 4 kq + 3)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16_t* vr = Vs + (dt * 16 + r16) * VP + c * 32 + 4 * kq;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vr + 16);
        const u32x4 vf = {a0[0], a0[1], a1[0], a1[1]};
        O[dt] = mfma_bf16(vf, pl[c], O[dt]);
        O[dt] = mfma_bf16(vf, ph[c], O[dt]);
      }
  };
  using I0 = std::integral_constant<int, 0>;
  load_step(0, I0{});
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();              // every wave is done reading the previous step
    store_step(I0{});
    __syncthreads();              // this step is staged
    if (s + 1 < nsteps) load_step(s + 1, I0{});   // in flight during the compute below
    if (owner) compute_step(s);
  }
  if (!owner) return;
  // chunk partial of query m: lane holds O^T[d = dt*16 + 4kq + e][m]
  float lt = lrun + __shfl_xor(lrun, 16);
  lt += __shfl_xor(lt, 32);
  if (m >= Mq) return;
  float* out = p.part + ((((size_t)l * nkv + g) * p.n_chunks + c) * 64 + m) * PW;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(out + dt * 16 + 4 * kq) = O[dt];
  if (kq == 0) { out[D] = mrun; out[D + 1] = lt; }
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
    float mr = -INFINITY;
    double lr = 0.0, o0 = 0.0, o1 = 0.0;
    for (int p0 = wb; p0 < we; p0 += 64) {
      const int pos = p0 + lane;
      const bool valid = pos < we && pos <= lim;
      float s = -INFINITY;
      if (valid) {
        const float* kr;
        if (pos < kvl) kr = Kp + (((size_t)clamp_blk(bt[pos >> 4], p.n_blocks) * nkv + g) * kBlock + (pos & 15)) * D;
        else kr = SK + ((size_t)(rs + pos - kvl) * nkv + g) * D;
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
        const float* vrow;
        size_t stride;
        if (vp < kvl) {
          vrow = Vp + ((size_t)clamp_blk(bt[vp >> 4], p.n_blocks) * nkv + g) * D * kBlock + (vp & 15);
          stride = kBlock;
        } else {
          vrow = SV + ((size_t)(rs + vp - kvl) * nkv + g) * D;
          stride = 1;
        }
        if (lane < D) o0 += pt * (double)vrow[(size_t)lane * stride];
        if (lane + 64 < D) o1 += pt * (double)vrow[(size_t)(lane + 64) * stride];
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
    out[(size_t)m * PW + dd] = (float)Oc;
    if (dd == 0) { out[(size_t)m * PW + D] = M; out[(size_t)m * PW + D + 1] = (float)Lc; }
  }
}

int launch_attention(const AttnParams& p, bool bf16, hipStream_t st) {
  dim3 grid(p.n_chunks, p.nkv, p.ri.L), block(256);
  if (bf16) {
    int maxMq = 0;
    for (int l = 0; l < p.ri.L; ++l) maxMq = p.ri.lane_cols[l] * p.G > maxMq ? p.ri.lane_cols[l] * p.G : maxMq;
    const int QT = (maxMq + 15) / 16;
    switch (QT) {
      case 1: hipLaunchKernelGGL(k_attn_bf16<1>, grid, block, 0, st, p); break;
      case 2: hipLaunchKernelGGL(k_attn_bf16<2>, grid, block, 0, st, p); break;
      case 3: hipLaunchKernelGGL(k_attn_bf16<3>, grid, block, 0, st, p); break;
      default: hipLaunchKernelGGL(k_attn_bf16<4>, grid, block, 0, st, p); break;
    }
  } else {
    int maxMq = 0;
    for (int l = 0; l < p.ri.L; ++l) maxMq = p.ri.lane_cols[l] * p.G > maxMq ? p.ri.lane_cols[l] * p.G : maxMq;
    const size_t lds = (size_t)4 * maxMq * (p.d + kAttnPartPad) * sizeof(float);
    hipLaunchKernelGGL(k_attn_f32, grid, block, lds, st, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Merge the chunk partials of each (lane, kv head) in chunk order; write o = O / L.
// Thread = (query row m, four consecutive d); all chunk loads of a thread are
// issued before the float64 merge, which visits the chunks in order.
constexpr int kCombineBatch = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnParams p, T* o) {
  const int g = blockIdx.x, l = blockIdx.y;
  const int D = p.d, PW = D + kAttnPartPad, DQ = D >> 2;
  const int mpw = blockDim.x / DQ;                       // query rows per workgroup
  const int m = blockIdx.z * mpw + threadIdx.x / DQ, dq = threadIdx.x - (threadIdx.x / DQ) * DQ;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int Mq = cols * p.G;
  if (threadIdx.x >= mpw * DQ || m >= Mq) return;
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int nch = min((end + p.chunk - 1) / p.chunk, p.n_chunks);
  const float* base = p.part + (((size_t)l * p.nkv + g) * p.n_chunks * 64 + m) * PW;
  const size_t cstride = (size_t)64 * PW;
  float M = -INFINITY;
  for (int c0 = 0; c0 < nch; c0 += kCombineBatch) {
    float mv[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) mv[i] = base[min(c0 + i, nch - 1) * cstride + D];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) M = fmaxf(M, mv[i]);
  }
  double Oc[4] = {0.0, 0.0, 0.0, 0.0}, Lc = 0.0;
  for (int c0 = 0; c0 < nch; c0 += kCombineBatch) {
    f32x4 ov[kCombineBatch];
    float mv[kCombineBatch], lv[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int c = min(c0 + i, nch - 1);
      const float* src = base + c * cstride;
      ov[i] = *reinterpret_cast<const f32x4*>(src + 4 * dq);
      mv[i] = src[D];
      lv[i] = src[D + 1];
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      if (c0 + i < nch && mv[i] != -INFINITY) {
        const double f = exp2((double)mv[i] - (double)M);
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
  const int mpw = 256 / (p.d / 4);
  dim3 grid(p.nkv, p.ri.L, (maxMq + mpw - 1) / mpw), block(256);
  if (bf16) hipLaunchKernelGGL(k_attn_combine<bf16_t>, grid, block, 0, st, p, reinterpret_cast<bf16_t*>(o));
  else hipLaunchKernelGGL(k_attn_combine<float>, grid, block, 0, st, p, reinterpret_cast<float*>(o));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
