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
// bf16 path (head_dim 128), per 32-position step:
//   S^T[pos][query] = K . Q^T with v_mfma_f32_16x16x32_bf16 (K rows = A, Q = B);
//   P = exp2(S * log2(e)/sqrt(d) - m) kept in fp32 and split into bf16 hi + lo
//   parts; O^T[d][query] += V^T . P_hi^T + V^T . P_lo^T.  The V pool is stored
//   d-major inside a block ([d][16 slots]) so that the V^T operand is read
//   straight from memory; the lane's key order inside the K = 32 MFMA step
//   equals the order in which the S^T result left it, so P needs no shuffle.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

template <int QT>
__global__ __launch_bounds__(256, 1) void k_attn_bf16(AttnParams p) {
  constexpr int D = 128, PW = D + 2;
  __shared__ float lds[4 * QT * 16 * PW];
  const int c = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kq = lane >> 4;
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
  const bf16_t* Qp = reinterpret_cast<const bf16_t*>(p.q);
  const bf16_t* Kp = reinterpret_cast<const bf16_t*>(p.kpool);
  const bf16_t* Vp = reinterpret_cast<const bf16_t*>(p.vpool);
  const bf16_t* SK = reinterpret_cast<const bf16_t*>(p.sk);
  const bf16_t* SV = reinterpret_cast<const bf16_t*>(p.sv);
  const int nkv = p.nkv;

  u32x4 qf[QT][4];
  int lim[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int m = qt * 16 + r16;
    if (m < Mq) {
      const int j = m / p.G, hh = m - j * p.G;
      const bf16_t* ptr = Qp + ((size_t)(rs + j) * p.nq + g * p.G + hh) * D + kq * 8;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[qt][ds] = *reinterpret_cast<const u32x4*>(ptr + ds * 32);
      lim[qt] = kvl + j;
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[qt][ds] = u32x4{0u, 0u, 0u, 0u};
      lim[qt] = -1;
    }
  }
  float mrun[QT], lrun[QT];
  f32x4 O[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY; lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int p0 = wb; p0 < we; p0 += 32) {
    // K rows of the two 16-position tiles: lane row = r16, d slice by kq
    u32x4 kf[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int pos = p0 + st * 16 + r16;
      const bf16_t* kp = nullptr;
      if (pos < kvl) {
        const int blk = clamp_blk(bt[pos >> 4], p.n_blocks);
        kp = Kp + (((size_t)blk * nkv + g) * kBlock + (pos & 15)) * D + kq * 8;
      } else if (pos < end) {
        kp = SK + ((size_t)(rs + pos - kvl) * nkv + g) * D + kq * 8;
      }
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        kf[st][ds] = kp ? *reinterpret_cast<const u32x4*>(kp + ds * 32) : u32x4{0u, 0u, 0u, 0u};
    }
    // V^T operand: lane row d = dt*16 + r16; keys 4kq..4kq+3 of each tile
    u32x4 vf[8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int base = p0 + st * 16;
      if (base + 16 <= kvl) {
        const int blk = clamp_blk(bt[base >> 4], p.n_blocks);
        const bf16_t* vp = Vp + (((size_t)blk * nkv + g) * D + r16) * kBlock + 4 * kq;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const u32x2 v2 = *reinterpret_cast<const u32x2*>(vp + (size_t)dt * 16 * kBlock);
          vf[dt][2 * st] = v2[0];
          vf[dt][2 * st + 1] = v2[1];
        }
      } else {
        const int blk = base < kvl ? clamp_blk(bt[base >> 4], p.n_blocks) : 0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int d = dt * 16 + r16;
          bf16_t e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = base + 4 * kq + e;
            bf16_t v = 0;
            if (pos < kvl) v = Vp[(((size_t)blk * nkv + g) * D + d) * kBlock + (pos & 15)];
            else if (pos < end) v = SV[((size_t)(rs + pos - kvl) * nkv + g) * D + d];
            e4[e] = v;
          }
          vf[dt][2 * st] = (uint32_t)e4[0] | ((uint32_t)e4[1] << 16);
          vf[dt][2 * st + 1] = (uint32_t)e4[2] | ((uint32_t)e4[3] << 16);
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x4 sc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        sc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) sc[st] = mfma_bf16(kf[st][ds], qf[qt][ds], sc[st]);
      }
      // lane holds S^T[p0 + 16 st + 4 kq + e][query qt*16 + r16]
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = p0 + st * 16 + 4 * kq + e;
          const float v = pos <= lim[qt] ? sc[st][e] * p.scale_log2 : -INFINITY;
          x[st * 4 + e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[qt], mx);
      float pr[8];
      float alpha = 1.f;
      if (mnew == -INFINITY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = 0.f;
      } else {
        alpha = exp2f(mrun[qt] - mnew);
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = exp2f(x[i] - mnew);
      }
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ps += pr[i];
      lrun[qt] = lrun[qt] * alpha + ps;
      mrun[qt] = mnew;
      u32x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16_t h0 = f2bf(pr[2 * i]), h1 = f2bf(pr[2 * i + 1]);
        const bf16_t l0 = f2bf(pr[2 * i] - bf2f(h0)), l1 = f2bf(pr[2 * i + 1] - bf2f(h1));
        ph[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        pl[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        O[qt][dt] *= alpha;
        O[qt][dt] = mfma_bf16(vf[dt], ph, O[qt][dt]);
        O[qt][dt] = mfma_bf16(vf[dt], pl, O[qt][dt]);
      }
    }
  }
  // wave partials -> LDS; lane holds O^T[d = dt*16 + 4kq + e][query qt*16 + r16]
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float lt = lrun[qt] + __shfl_xor(lrun[qt], 16);
    lt += __shfl_xor(lt, 32);
    const int m = qt * 16 + r16;
    float* dst = lds + ((size_t)wave * QT * 16 + m) * PW;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[dt * 16 + 4 * kq + e] = O[qt][dt][e];
    if (kq == 0) { dst[D] = mrun[qt]; dst[D + 1] = lt; }
  }
  __syncthreads();
  float* out = p.part + (((size_t)l * nkv + g) * p.n_chunks + c) * 64 * PW;
  for (int idx = threadIdx.x; idx < Mq * D; idx += blockDim.x) {
    const int m = idx >> 7, dd = idx & (D - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds[((size_t)w * QT * 16 + m) * PW + D]);
    float Oc = 0.f, Lc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* src = lds + ((size_t)w * QT * 16 + m) * PW;
        if (src[D] != -INFINITY) {
          const float f = exp2f(src[D] - M);
          Oc += src[dd] * f;
          Lc += src[D + 1] * f;
        }
      }
    }
    out[(size_t)m * PW + dd] = Oc;
    if (dd == 0) { out[(size_t)m * PW + D] = M; out[(size_t)m * PW + D + 1] = Lc; }
  }
}

// fp32 model: VALU, one query row at a time per wave, 64 positions per step (lane = position).
__global__ __launch_bounds__(256) void k_attn_f32(AttnParams p) {
  extern __shared__ float lds[];   // [4][Mq][d + 2]
  const int c = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int D = p.d, PW = D + 2;
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
    float mr = -INFINITY, lr = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p0 = wb; p0 < we; p0 += 64) {
      const int pos = p0 + lane;
      const bool valid = pos < we && pos <= lim;
      float s = -INFINITY;
      if (valid) {
        const float* kr;
        if (pos < kvl) kr = Kp + (((size_t)clamp_blk(bt[pos >> 4], p.n_blocks) * nkv + g) * kBlock + (pos & 15)) * D;
        else kr = SK + ((size_t)(rs + pos - kvl) * nkv + g) * D;
        float a = 0.f;
        for (int i = 0; i < D; ++i) a = fmaf(q[i], kr[i], a);
        s = a * p.scale_log2;
      }
      const float mx = wave_max(s);
      const float mnew = fmaxf(mr, mx);
      if (mnew == -INFINITY) continue;
      const float alpha = exp2f(mr - mnew);
      const float pr = valid ? exp2f(s - mnew) : 0.f;
      lr = lr * alpha + wave_sum(pr);
      o0 *= alpha; o1 *= alpha;
      const int nval = min(64, we - p0);
      for (int t = 0; t < nval; ++t) {
        const float pt = __shfl(pr, t);
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
        if (lane < D) o0 = fmaf(pt, vrow[(size_t)lane * stride], o0);
        if (lane + 64 < D) o1 = fmaf(pt, vrow[(size_t)(lane + 64) * stride], o1);
      }
      mr = mnew;
    }
    float* dst = lds + ((size_t)wave * Mq + m) * PW;
    if (lane < D) dst[lane] = o0;
    if (lane + 64 < D) dst[lane + 64] = o1;
    if (lane == 0) { dst[D] = mr; dst[D + 1] = lr; }
  }
  __syncthreads();
  float* out = p.part + (((size_t)l * nkv + g) * p.n_chunks + c) * 64 * PW;
  for (int idx = threadIdx.x; idx < Mq * D; idx += blockDim.x) {
    const int m = idx / D, dd = idx - m * D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds[((size_t)w * Mq + m) * PW + D]);
    float Oc = 0.f, Lc = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float* src = lds + ((size_t)w * Mq + m) * PW;
        if (src[D] != -INFINITY) {
          const float f = exp2f(src[D] - M);
          Oc += src[dd] * f;
          Lc += src[D + 1] * f;
        }
      }
    }
    out[(size_t)m * PW + dd] = Oc;
    if (dd == 0) { out[(size_t)m * PW + D] = M; out[(size_t)m * PW + D + 1] = Lc; }
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
    const size_t lds = (size_t)4 * maxMq * (p.d + 2) * sizeof(float);
    hipLaunchKernelGGL(k_attn_f32, grid, block, lds, st, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Merge the chunk partials of each (lane, kv head) in chunk order; write o = O / L.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnParams p, T* o) {
  const int g = blockIdx.x, l = blockIdx.y;
  const int D = p.d, PW = D + 2;
  const int cols = p.ri.lane_cols[l], rs = p.ri.lane_start[l];
  const int cap = p.max_blocks * kBlock;
  const int kvl = max(0, min(p.kv_len[l], cap - cols));
  const int end = kvl + cols;
  const int nch = min((end + p.chunk - 1) / p.chunk, p.n_chunks);
  const int Mq = cols * p.G;
  const float* base = p.part + (((size_t)l * p.nkv + g) * p.n_chunks) * 64 * PW;
  for (int idx = threadIdx.x; idx < Mq * D; idx += blockDim.x) {
    const int m = idx / D, dd = idx - m * D;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, base[((size_t)c * 64 + m) * PW + D]);
    float Oc = 0.f, Lc = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float* src = base + ((size_t)c * 64 + m) * PW;
      if (src[D] != -INFINITY) {
        const float f = exp2f(src[D] - M);
        Oc += src[dd] * f;
        Lc += src[D + 1] * f;
      }
    }
    const int j = m / p.G, hh = m - j * p.G;
    st_act(o + ((size_t)(rs + j) * p.nq + g * p.G + hh) * D + dd, Oc / Lc);
  }
}

int launch_attn_combine(const AttnParams& p, void* o, bool bf16, hipStream_t st) {
  dim3 grid(p.nkv, p.ri.L), block(256);
  if (bf16) hipLaunchKernelGGL(k_attn_combine<bf16_t>, grid, block, 0, st, p, reinterpret_cast<bf16_t*>(o));
  else hipLaunchKernelGGL(k_attn_combine<float>, grid, block, 0, st, p, reinterpret_cast<float*>(o));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
