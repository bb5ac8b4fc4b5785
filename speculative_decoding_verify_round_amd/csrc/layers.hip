// Per-row layer kernels of the verify round and the commit (gfx950).
//
//   embed + RMSNorm, split-K reduce + residual + RMSNorm, the RoPE table,
//   QKV post-processing (rotation, rounding, K/V staging), the gated-delta-rule
//   column recurrence (verify) and its replay (commit), and the KV compaction.
//
// Commit follows "Speculative decoding" (gpillon.github.io/ignis), step 5: the
// state moves forward by exactly the committed run; attention layers keep the
// keys of every committed column and recurrent layers replay only the
// committed prefix, so a rejected column leaves no trace.  The FreeToken
// tracking issue ("Per-request state") fixes the split: verify only reads the
// live state and stages scratch, commit rolls the state to the accepted count.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

// ------------------------------------------------------------------------------- RoPE table
// cos/sin of pos * theta^(-2i/d) for every row, in double precision.
__global__ void k_rope_table(const int32_t* kv_len, RowInfo ri, int d, double theta, double* table) {
  const int r = blockIdx.x, i = threadIdx.x;
  if (i >= d / 2) return;
  const int l = ri.row_lane[r];
  const double pos = (double)(kv_len[l] + ri.row_col[r]);
  const double ang = pos * pow(theta, -2.0 * (double)i / (double)d);
  table[((size_t)r * (d / 2) + i) * 2 + 0] = cos(ang);
  table[((size_t)r * (d / 2) + i) * 2 + 1] = sin(ang);
}

int launch_rope_table(const int32_t* kv_len, const RowInfo& ri, int d, float theta, double* table,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_rope_table, dim3(ri.R), dim3(64), 0, st, kv_len, ri, d, (double)theta, table);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- RMSNorm family
// One 1024-thread workgroup per row; thread t owns the float4 groups t and
// t + 1024 of the row (hidden <= 8192) and issues all of its loads before it
// uses any.  h = float32(x / sqrt(mean(x^2) + eps) * gain), evaluated in
// float64; a bf16 model stores h as hi/lo bf16 planes in fragment order.
constexpr int kRowThreads = 1024;
constexpr int kRowGroups = 2;     // float4 groups per thread
constexpr int kSplitBatch = 8;    // split partials loaded per batch

template <typename T>
__device__ __forceinline__ void norm_store(const f32x4 (&xn)[kRowGroups], int r, int H, const float* gain, float eps,
                                           T* h, size_t plane, double ss, double* red) {
  const double tot = block_sum_f64(ss, red);
  const double scale = 1.0 / sqrt(tot / (double)H + (double)eps);
#pragma unroll
  for (int gi = 0; gi < kRowGroups; ++gi) {
    const int g = threadIdx.x + gi * kRowThreads;
    if (4 * g >= H) break;
    const f32x4 gn = *reinterpret_cast<const f32x4*>(gain + 4 * g);
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)((double)xn[gi][e] * scale * (double)gn[e]);
    st_out4(h, plane, r, 4 * g, H, v);
  }
}

__device__ __forceinline__ f32x4 ld_act4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld_act4(const bf16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
               __uint_as_float(w[1] & 0xffff0000u)};
}

// Also zeroes the nzero arrival counters of the round's balanced gate/up launches
// (each launch leaves them zero again; this covers a workspace that held anything else).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_embed_norm(const int32_t* tokens, const T* embed, int V, int H,
                                                             const float* gain, float eps, float* x, T* h, int R,
                                                             int* zero, int nzero) {
  __shared__ double red[32];
  const int r = blockIdx.x;
  if (r == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  int tok = tokens[r];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  float* xr = x + (size_t)r * H;
  const T* e = embed + (size_t)tok * H;
  f32x4 xn[kRowGroups];
  double ss = 0.0;
#pragma unroll
  for (int gi = 0; gi < kRowGroups; ++gi) {
    const int g = threadIdx.x + gi * kRowThreads;
    xn[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (4 * g >= H) continue;
    xn[gi] = ld_act4(e + 4 * g);
    *reinterpret_cast<f32x4*>(xr + 4 * g) = xn[gi];
#pragma unroll
    for (int q = 0; q < 4; ++q) ss += (double)xn[gi][q] * (double)xn[gi][q];
  }
  norm_store(xn, r, H, gain, eps, h, act_plane(R, H), ss, red);
}

int launch_embed_norm(const int32_t* tokens, const void* embed, int V, int H, const float* gain, float eps,
                      float* x, void* h, const RowInfo& ri, bool bf16, int* zero, int nzero, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(k_embed_norm<bf16_t>, dim3(ri.R), dim3(kRowThreads), 0, st, tokens,
                       reinterpret_cast<const bf16_t*>(embed), V, H, gain, eps, x, reinterpret_cast<bf16_t*>(h), ri.R,
                       zero, nzero);
  else
    hipLaunchKernelGGL(k_embed_norm<float>, dim3(ri.R), dim3(kRowThreads), 0, st, tokens,
                       reinterpret_cast<const float*>(embed), V, H, gain, eps, x, reinterpret_cast<float*>(h), ri.R,
                       zero, nzero);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Sum of the S split partials of one float4 of a projection, in split order, in float64.
// A batch's splits past S are loaded (clamped to split S - 1) and dropped by selects, not
// branches: a branch lets the compiler sink each load to its addition, one memory round
// trip per split.
__device__ __forceinline__ void sum_splits4(const float* P, size_t split_stride, int S, double (&t)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = 0.0;
  for (int s0 = 0; s0 < S; s0 += kSplitBatch) {
    f32x4 pv[kSplitBatch];
#pragma unroll
    for (int i = 0; i < kSplitBatch; ++i)
      pv[i] = *reinterpret_cast<const f32x4*>(P + (size_t)min(s0 + i, S - 1) * split_stride);
#pragma unroll
    for (int i = 0; i < kSplitBatch; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        t[e] = s0 + i == 0 ? (double)pv[i][e] : s0 + i < S ? t[e] + (double)pv[i][e] : t[e];
  }
}

// The first kSplitBatch split partials of four consecutive floats, loaded (clamped to a
// valid split) and then summed in split order in float64: callers issue every load of a
// thread before the first sum.
__device__ __forceinline__ void load_splits4(const float* P, size_t split_stride, int S, f32x4 (&pv)[kSplitBatch]) {
#pragma unroll
  for (int i = 0; i < kSplitBatch; ++i) pv[i] = *reinterpret_cast<const f32x4*>(P + (size_t)min(i, S - 1) * split_stride);
}
__device__ __forceinline__ void sum_loaded4(const f32x4 (&pv)[kSplitBatch], const float* P, size_t split_stride, int S,
                                            double (&t)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = (double)pv[0][e];
#pragma unroll
  for (int i = 1; i < kSplitBatch; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = i < S ? t[e] + (double)pv[i][e] : t[e];
  if (S > kSplitBatch) {   // more splits than one batch (the split rule caps the inputs at four)
    double u[4];
    sum_splits4(P + kSplitBatch * split_stride, split_stride, S - kSplitBatch, u);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] += u[e];
  }
}

// x[r] += float(sum_s P[s][r]) (s in order), then h[r] = round(rmsnorm(x[r]) * gain).
// Every load of the row (residual, the S partials, the gains of both float4 groups) is
// issued before the first is used, so the kernel pays one memory round trip; S is a
// template argument so that no lane loads a split twice.
template <typename T, int S>
__global__ __launch_bounds__(kRowThreads) void k_resid_norm(const float* P, int R, float* x, int H,
                                                             const float* gain, float eps, T* h) {
  __shared__ double red[32];
  const int r = blockIdx.x;
  float* xr = x + (size_t)r * H;
  const size_t sstride = (size_t)R * H;
  f32x4 xo[kRowGroups], gn[kRowGroups], pv[kRowGroups][S];
#pragma unroll
  for (int gi = 0; gi < kRowGroups; ++gi) {
    const int g = min(threadIdx.x + gi * (int)blockDim.x, H / 4 - 1);   // a valid address for every lane
    xo[gi] = *reinterpret_cast<const f32x4*>(xr + 4 * g);
    gn[gi] = *reinterpret_cast<const f32x4*>(gain + 4 * g);
#pragma unroll
    for (int b = 0; b < S; ++b) pv[gi][b] = *reinterpret_cast<const f32x4*>(P + (size_t)r * H + 4 * g + b * sstride);
  }
  // every group is summed (a clamped group repeats the row's last one) and only valid
  // groups are stored and counted: no branch between the loads and their use
  f32x4 xn[kRowGroups];
  double ss = 0.0;
#pragma unroll
  for (int gi = 0; gi < kRowGroups; ++gi) {
    const int g = threadIdx.x + gi * (int)blockDim.x;
    const bool ok = 4 * g < H;
    double t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (double)pv[gi][0][e];
#pragma unroll
    for (int b = 1; b < S; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] += (double)pv[gi][b][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) xn[gi][e] = (float)((double)xo[gi][e] + (double)(float)t[e]);   // x + float(projection)
    if (ok) *reinterpret_cast<f32x4*>(xr + 4 * g) = xn[gi];
#pragma unroll
    for (int q = 0; q < 4; ++q) ss += ok ? (double)xn[gi][q] * (double)xn[gi][q] : 0.0;
  }
  const double tot = block_sum_f64(ss, red);
  const double scale = 1.0 / sqrt(tot / (double)H + (double)eps);
  const size_t plane = act_plane(R, H);
#pragma unroll
  for (int gi = 0; gi < kRowGroups; ++gi) {
    const int g = threadIdx.x + gi * (int)blockDim.x;
    if (4 * g >= H) break;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)((double)xn[gi][e] * scale * (double)gn[gi][e]);
    st_out4(h, plane, r, 4 * g, H, v);
  }
}

// Threads of a row's workgroup: just enough for kRowGroups float4 groups each (whole
// waves).  Every load instruction costs the address unit the same time whether or not its
// lanes need it, and one workgroup per row leaves most of a round's 64 rows on one CU each.
static int row_threads(int H) {
  const int t = ((H / 4 + kRowGroups - 1) / kRowGroups + 63) / 64 * 64;
  return t < kRowThreads ? t : kRowThreads;
}

int launch_resid_norm(const float* P, int S, float* x, int H, const float* gain, float eps, void* h,
                      const RowInfo& ri, bool bf16, hipStream_t st) {
  if (H / 4 > kRowGroups * kRowThreads || S < 1 || S > kSplitBatch) return -1;
  const dim3 block(row_threads(H));
  const void* f = nullptr;
#define SV_RN(S_) f = bf16 ? reinterpret_cast<const void*>(&k_resid_norm<bf16_t, S_>) \
                         : reinterpret_cast<const void*>(&k_resid_norm<float, S_>)
  switch (S) {
    case 1: SV_RN(1); break;
    case 2: SV_RN(2); break;
    case 3: SV_RN(3); break;
    case 4: SV_RN(4); break;
    case 5: SV_RN(5); break;
    case 6: SV_RN(6); break;
    case 7: SV_RN(7); break;
    default: SV_RN(8); break;
  }
#undef SV_RN
  int R = ri.R;
  void* args[] = {&P, &R, &x, &H, &gain, &eps, &h};
  if (hipLaunchKernel(f, dim3(ri.R), block, args, 0, st) != hipSuccess) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- QKV post
// Sum the split-K partials of [q | k | v], rotate q and k (rotate-half, pair (i, i + d/2)),
// round to the storage type, write q and stage K/V of every column.  One 1024-thread
// workgroup per row; a thread takes four consecutive pairs of a q or k head, or four
// consecutive v elements, and loads all splits before summing them.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_qkv_post(const float* P, int S, RowInfo ri, const double* rope,
                                                           int use_rope, int nq, int nkv, int d, float* q, T* sk,
                                                           T* sv, KvStage ks) {
  const int R = ri.R;
  if ((int)blockIdx.x >= R) {
    // The lane's staged slots that are not its own columns: the committed prefix of the
    // first staged block (K and V) and zeros after the last column (V; K there is masked
    // and never meets a nonzero weight).  Every load is issued (from a valid address)
    // before the first store.
    const int l = blockIdx.x - R, cols = ri.lane_cols[l];
    const int kvl = max(0, min(ks.kv_len[l], ks.max_blocks * kBlock - cols));
    const int pre = kvl & 15;
    const int blk = clamp_blk(ks.block_table[(size_t)l * ks.max_blocks + (kvl >> 4)], ks.n_blocks);
    const T* Kc = reinterpret_cast<const T*>(ks.kpool);
    const T* Vc = reinterpret_cast<const T*>(ks.vpool);
    const size_t sb0 = (size_t)kStageBlocks * l;
    constexpr int E = 16 / sizeof(T);            // elements per 16-byte chunk
    typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));
    // K prefix: thread = (head, slot < 16, 16-byte chunk of the d row)
    const int kchunks = nkv * kBlock * (d / E);
    for (int it = threadIdx.x; it < kchunks; it += blockDim.x) {
      const int c = it % (d / E), gs = it / (d / E), sp = gs % kBlock, g = gs / kBlock;
      const size_t o = ((size_t)g * kBlock + sp) * d + c * E;
      const chunk_t v = *reinterpret_cast<const chunk_t*>(Kc + (size_t)blk * nkv * kBlock * d + o);
      if (sp < pre) *reinterpret_cast<chunk_t*>(sk + sb0 * nkv * kBlock * d + o) = v;
    }
    // V rows: thread = (head, d); slots [0, pre) from the cache, [pre + cols, 32) zero,
    // written in whole 16-byte groups except where a group holds own columns
    for (int it = threadIdx.x; it < nkv * d; it += blockDim.x) {
      const int g = it / d, i = it - g * d;
      const T* vrow = Vc + (((size_t)blk * nkv + g) * d + i) * kBlock;
      T row[kBlock];
#pragma unroll
      for (int h = 0; h < kBlock / E; ++h) *reinterpret_cast<chunk_t*>(row + h * E) = *reinterpret_cast<const chunk_t*>(vrow + h * E);
#pragma unroll
      for (int grp = 0; grp < kStageBlocks * kBlock / E; ++grp) {
        const int s0 = grp * E;
        T* dst = sv + (((sb0 + s0 / kBlock) * nkv + g) * d + i) * kBlock + (s0 % kBlock);
        T w[E];
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] = s0 + e < pre ? row[(s0 + e) % kBlock] : T(0);
        if (s0 + E <= pre || s0 >= pre + cols) {
          *reinterpret_cast<chunk_t*>(dst) = *reinterpret_cast<const chunk_t*>(w);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (s0 + e < pre || s0 + e >= pre + cols) dst[e] = w[e];
        }
      }
    }
    return;
  }
  const int r = blockIdx.x;
  const int l = ri.row_lane[r], j = ri.row_col[r], cols = ri.lane_cols[l];
  const int kvl = max(0, min(ks.kv_len[l], ks.max_blocks * kBlock - cols));
  const int pre = kvl & 15, slot = pre + j;   // column j sits at position kvl + j: staged block slot / 16
  const size_t sb = (size_t)kStageBlocks * l + (slot >> 4);
  const int sl = slot & 15;
  const int N = (nq + 2 * nkv) * d, half = d / 2;
  const size_t sstride = (size_t)R * N;
  const float* Pr = P + (size_t)r * N;
  const int nrot = (nq + nkv) * (half / 4), nv = nkv * d / 4;
  for (int it = threadIdx.x; it < nrot + nv; it += blockDim.x) {
    if (it < nrot) {
      const int hd = it / (half / 4), i0 = 4 * (it - hd * (half / 4));
      double a[4], b[4];
      sum_splits4(Pr + hd * d + i0, sstride, S, a);
      sum_splits4(Pr + hd * d + i0 + half, sstride, S, b);
      float ra[4], rb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double av = (double)(float)a[e], bv = (double)(float)b[e];   // the projection, rounded once
        double x = av, y = bv;
        if (use_rope) {
          const double c = rope[((size_t)r * half + i0 + e) * 2], sn = rope[((size_t)r * half + i0 + e) * 2 + 1];
          x = av * c - bv * sn;
          y = bv * c + av * sn;
        }
        ra[e] = (float)x;
        rb[e] = (float)y;
      }
      if (hd < nq) {
        float* dst = q + ((size_t)r * nq + hd) * d;
        *reinterpret_cast<f32x4*>(dst + i0) = f32x4{ra[0], ra[1], ra[2], ra[3]};
        *reinterpret_cast<f32x4*>(dst + i0 + half) = f32x4{rb[0], rb[1], rb[2], rb[3]};
      } else {
        T* dst = sk + ((sb * nkv + (hd - nq)) * kBlock + sl) * d;     // staged for the cache
#pragma unroll
        for (int e = 0; e < 4; ++e) { st_act(dst + i0 + e, ra[e]); st_act(dst + i0 + half + e, rb[e]); }
      }
    } else {
      const int i0 = 4 * (it - nrot);
      double v[4];
      sum_splits4(Pr + (nq + nkv) * d + i0, sstride, S, v);
      const int g = i0 / d, i = i0 - g * d;   // d % 4 == 0: the four elements share a head
#pragma unroll
      for (int e = 0; e < 4; ++e) st_act(sv + ((sb * nkv + g) * d + i + e) * kBlock + sl, (float)(double)(float)v[e]);
    }
  }
}

int launch_qkv_post(const float* P, int S, const double* rope, int use_rope, int nq, int nkv, int d,
                    float* q, void* sk, void* sv, const KvStage& ks, const RowInfo& ri, bool bf16, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(k_qkv_post<bf16_t>, dim3(ri.R + ri.L), dim3(kRowThreads), 0, st, P, S, ri, rope, use_rope, nq, nkv, d,
                       q, reinterpret_cast<bf16_t*>(sk), reinterpret_cast<bf16_t*>(sv), ks);
  else
    hipLaunchKernelGGL(k_qkv_post<float>, dim3(ri.R + ri.L), dim3(kRowThreads), 0, st, P, S, ri, rope, use_rope, nq, nkv, d,
                       q, reinterpret_cast<float*>(sk), reinterpret_cast<float*>(sv), ks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- gated delta rule
// State S is [dv][dk] float32 per (lane, head).  One column step (Yang et al., Gated
// DeltaNet), evaluated in float64 and stored in float32 after every column:
//   S <- alpha S + beta (v - alpha S k) k^T,   o = S q.
// Row i of the new state depends only on row i of the old one and on the column's
// shared k, v_i, alpha, beta, so rows split freely: kGdnRowBlocks workgroups per (lane,
// head) of kGdnRows rows each, eight threads per row holding sixteen entries of it.  Verify
// and commit run the same step function on the same float32 inputs (the verify stages
// them), so the committed state is bitwise the state verify saw at the last committed
// column.
constexpr int kGdnDim = 128;
constexpr int kGdnRowBlocks = 4;
constexpr int kGdnRows = kGdnDim / kGdnRowBlocks;   // 32 rows: 256 threads, 8 per row
constexpr int kGdnSeg = kGdnDim / 8;                // 16 entries per thread

// S[i,:] . vec over the eight threads of row i (entries 16 seg .. 16 seg + 15 each),
// summed in a fixed tree; every thread of the row gets the same bits (a + b == b + a).
__device__ __forceinline__ double gdn_dot(const float (&s)[kGdnSeg], const float* vec, int seg) {
  double part = 0.0;
#pragma unroll
  for (int e = 0; e < kGdnSeg; ++e) part += (double)s[e] * (double)vec[kGdnSeg * seg + e];
  part += __shfl_xor(part, 1);
  part += __shfl_xor(part, 2);
  part += __shfl_xor(part, 4);
  return part;
}

__device__ __forceinline__ void gdn_step(float (&s)[kGdnSeg], const float* k, int seg, double v_i, double alpha,
                                         double beta) {
  const double coef = beta * (v_i - alpha * gdn_dot(s, k, seg));
#pragma unroll
  for (int e = 0; e < kGdnSeg; ++e) s[e] = (float)(alpha * (double)s[e] + coef * (double)k[kGdnSeg * seg + e]);
}

// stage layout per (row, head): kn[128], v[128], alpha, beta  (kGdnStage floats)
constexpr int kGdnStage = 2 * kGdnDim + 2;

// The row's state slice: row i, entries 16 seg .. 16 seg + 15.
__device__ __forceinline__ const float* gdn_slice(const float* state, int l, int n_gdn, int gi, int hg, int h, int row,
                                                  int seg) {
  return state + ((((size_t)l * n_gdn + gi) * hg + h) * kGdnDim + row) * kGdnDim + kGdnSeg * seg;
}

// Verify of one layer: workgroup (row block, head, lane).  First every column's inputs --
// the projection's split partials summed in split order in float64 and rounded once;
// q and k L2-normalised (q scaled by d^-1/2), alpha = sigmoid, beta = sigmoid -- into
// LDS, with the norms reduced over 32 lanes in a fixed tree; then the columns one after
// another with no further barrier.  The state is read, never written.
template <typename T>
__global__ __launch_bounds__(256) void k_gdn_verify(const float* P, int S, RowInfo ri, int hg, const float* state,
                                                     int n_gdn, int gi, float* stage, T* o) {
  __shared__ float sq[kMaxCols][kGdnDim], sk[kMaxCols][kGdnDim], sv[kMaxCols][kGdnRows], sab[kMaxCols][2];
  const int rb = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int t = threadIdx.x, row = rb * kGdnRows + (t >> 3), seg = t & 7;
  const int R = ri.R, N = 3 * hg * kGdnDim + 2 * hg;
  const int cols = ri.lane_cols[l], rs = ri.lane_start[l];
  const size_t split = (size_t)R * N;
  float s[kGdnSeg];
  {
    const float* S0 = gdn_slice(state, l, n_gdn, gi, hg, h, row, seg);
#pragma unroll
    for (int e = 0; e < kGdnSeg; e += 4) {
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(S0 + e);
      s[e] = v4[0]; s[e + 1] = v4[1]; s[e + 2] = v4[2]; s[e + 3] = v4[3];
    }
  }
  // q and k: 64 four-element items per column, 32 consecutive threads per vector; v of
  // the block's rows: eight items per column; alpha and beta: two per column.  The
  // thread's first item of each kind has its splits loaded together with the state, so
  // rounds of up to four columns wait for memory once; later q/k items load their own.
  const int nqk = cols * 64, nv = cols * (kGdnRows / 4), nab = 2 * cols;
  auto qk_src = [&](int it) {
    const int j = it >> 6, vec = (it >> 5) & 1, quad = it & 31;
    return P + (size_t)(rs + j) * N + vec * hg * kGdnDim + h * kGdnDim + 4 * quad;
  };
  auto v_src = [&](int it) {
    const int j = it / (kGdnRows / 4), quad = it % (kGdnRows / 4);
    return P + (size_t)(rs + j) * N + 2 * hg * kGdnDim + h * kGdnDim + rb * kGdnRows + 4 * quad;
  };
  f32x4 pqk[kSplitBatch], pvv[kSplitBatch];
  float pab[kSplitBatch];
  load_splits4(qk_src(min(t, nqk - 1)), split, S, pqk);
  load_splits4(v_src(min(t, nv - 1)), split, S, pvv);
  {
    const int i = min(t, nab - 1), j = i >> 1, w = i & 1;
    const float* src = P + (size_t)(rs + j) * N + 3 * hg * kGdnDim + w * hg + h;
#pragma unroll
    for (int b = 0; b < kSplitBatch; ++b) pab[b] = src[(size_t)min(b, S - 1) * split];
  }
  auto qk_item = [&](int it, const double (&a)[4]) {   // uniform over each 32-thread group
    const int j = it >> 6, vec = (it >> 5) & 1, quad = it & 31;
    float f[4];
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = (float)a[e];
      ss += (double)f[e] * (double)f[e];
    }
#pragma unroll
    for (int x = 1; x <= 16; x <<= 1) ss += __shfl_xor(ss, x);
    const double inv = 1.0 / sqrt(ss + 1e-6);
    float* dst = vec ? &sk[j][4 * quad] : &sq[j][4 * quad];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dst[e] = vec ? (float)((double)f[e] * inv) : (float)((double)f[e] * inv / sqrt((double)kGdnDim));
  };
  if (t < nqk) {
    double a[4];
    sum_loaded4(pqk, qk_src(t), split, S, a);
    qk_item(t, a);
  }
  for (int it = t + 256; it < nqk; it += 256) {
    double a[4];
    sum_splits4(qk_src(it), split, S, a);
    qk_item(it, a);
  }
  if (t < nv) {
    double a[4];
    sum_loaded4(pvv, v_src(t), split, S, a);
    const int j = t / (kGdnRows / 4), quad = t % (kGdnRows / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[j][4 * quad + e] = (float)a[e];
  }
  if (t < nab) {
    double a = (double)pab[0];
#pragma unroll
    for (int b = 1; b < kSplitBatch; ++b) a = b < S ? a + (double)pab[b] : a;
    sab[t >> 1][t & 1] = (float)(1.0 / (1.0 + exp(-(double)(float)a)));
  }
  __syncthreads();
  // stage the column inputs for the commit's replay: k, alpha, beta once (row block 0),
  // v of each block's own rows
  for (int it = t; it < cols * kGdnDim; it += 256) {
    const int j = it / kGdnDim, e = it % kGdnDim;
    float* stg = stage + ((size_t)(rs + j) * hg + h) * kGdnStage;
    if (rb == 0) stg[e] = sk[j][e];
    if (e < kGdnRows) stg[kGdnDim + rb * kGdnRows + e] = sv[j][e];
    if (rb == 0 && e < 2) stg[2 * kGdnDim + e] = sab[j][e];
  }
  const size_t oplane = act_plane(R, hg * kGdnDim);
  for (int j = 0; j < cols; ++j) {
    gdn_step(s, sk[j], seg, (double)sv[j][t >> 3], (double)sab[j][0], (double)sab[j][1]);
    const double oi = gdn_dot(s, sq[j], seg);
    if (seg == 0) st_out(o, oplane, act_index(o, rs + j, h * kGdnDim + row, hg * kGdnDim), (float)oi);
  }
}

int launch_gdn_verify(const float* P, int S, int hg, int dg, const float* state, int n_gdn, int gi,
                      float* stage, void* o, const RowInfo& ri, bool bf16, hipStream_t st) {
  (void)dg;
  dim3 grid(kGdnRowBlocks, hg, ri.L), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_gdn_verify<bf16_t>, grid, block, 0, st, P, S, ri, hg, state, n_gdn, gi, stage,
                       reinterpret_cast<bf16_t*>(o));
  else
    hipLaunchKernelGGL(k_gdn_verify<float>, grid, block, 0, st, P, S, ri, hg, state, n_gdn, gi, stage,
                       reinterpret_cast<float*>(o));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Commit: replay columns 0 .. c-1 of every gated-delta-rule layer from the staged inputs,
// workgroup (row block, head) x lane x layer, the same step function as the verify.
__global__ __launch_bounds__(256) void k_gdn_replay(const int32_t* committed, float* state, int n_gdn, int hg,
                                                     const float* stage, size_t stage_layer_stride, RowInfo ri) {
  __shared__ float sk[kMaxCols][kGdnDim], sv[kMaxCols][kGdnRows], sab[kMaxCols][2];
  const int rb = blockIdx.x % kGdnRowBlocks, h = blockIdx.x / kGdnRowBlocks, l = blockIdx.y, gi = blockIdx.z;
  const int t = threadIdx.x, row = rb * kGdnRows + (t >> 3), seg = t & 7;
  const int cols = ri.lane_cols[l], rs = ri.lane_start[l];
  const int c = max(1, min(committed[l], cols));
  float* S0 = const_cast<float*>(gdn_slice(state, l, n_gdn, gi, hg, h, row, seg));
  float s[kGdnSeg];
#pragma unroll
  for (int e = 0; e < kGdnSeg; e += 4) {
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(S0 + e);
    s[e] = v4[0]; s[e + 1] = v4[1]; s[e + 2] = v4[2]; s[e + 3] = v4[3];
  }
  const float* stl = stage + gi * stage_layer_stride;
  for (int it = t; it < c * (kGdnDim / 4); it += 256) {
    const int j = it / (kGdnDim / 4), quad = it % (kGdnDim / 4);
    const float* stg = stl + ((size_t)(rs + j) * hg + h) * kGdnStage;
    const f32x4 k4 = *reinterpret_cast<const f32x4*>(stg + 4 * quad);
#pragma unroll
    for (int e = 0; e < 4; ++e) sk[j][4 * quad + e] = k4[e];
    if (quad < kGdnRows / 4) {
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(stg + kGdnDim + rb * kGdnRows + 4 * quad);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[j][4 * quad + e] = v4[e];
    }
    if (quad < 2) sab[j][quad] = stg[2 * kGdnDim + quad];
  }
  __syncthreads();
  for (int j = 0; j < c; ++j) gdn_step(s, sk[j], seg, (double)sv[j][t >> 3], (double)sab[j][0], (double)sab[j][1]);
#pragma unroll
  for (int e = 0; e < kGdnSeg; e += 4) *reinterpret_cast<f32x4*>(S0 + e) = f32x4{s[e], s[e + 1], s[e + 2], s[e + 3]};
}

int launch_gdn_replay(const int32_t* committed, float* state, int n_gdn, int hg, int dg, const float* stage,
                      size_t stage_layer_stride, const RowInfo& ri, hipStream_t st) {
  (void)dg;
  dim3 grid(kGdnRowBlocks * hg, ri.L, n_gdn), block(256);
  hipLaunchKernelGGL(k_gdn_replay, grid, block, 0, st, committed, state, n_gdn, hg, stage, stage_layer_stride, ri);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------------------- KV compaction
// Staged K/V of columns 0 .. c-1 (staged block slots kv_len % 16 + j) -> paged cache at
// positions kv_len .. kv_len + c - 1.
// K blocks are [slot][d], V blocks are [d][slot].
template <typename T>
__global__ __launch_bounds__(256) void k_commit_kv(const int32_t* committed, const int32_t* kv_len,
                                                    const int32_t* block_table, int max_blocks, int n_blocks,
                                                    T* kpool, T* vpool, int nkv, int d, const T* sk, const T* sv,
                                                    size_t stage_layer_elems, RowInfo ri) {
  const int l = blockIdx.x, li = blockIdx.y;
  const int cols = ri.lane_cols[l];
  const int c = max(1, min(committed[l], cols));
  const int cap = max_blocks * kBlock;
  const int kvl = max(0, min(kv_len[l], cap - cols));
  const size_t layer_pool = (size_t)n_blocks * nkv * kBlock * d;
  T* kp = kpool + li * layer_pool;
  T* vp = vpool + li * layer_pool;
  const T* skl = sk + li * stage_layer_elems;
  const T* svl = sv + li * stage_layer_elems;
  const int per_col = nkv * d, n = c * per_col;
  // the committed columns span at most two cache blocks: their ids are read once
  const int* btl = block_table + (size_t)l * max_blocks;
  const int blk0 = clamp_blk(btl[kvl >> 4], n_blocks);
  const int blk1 = clamp_blk(btl[min((kvl + c - 1) >> 4, max_blocks - 1)], n_blocks);
  // kU elements per thread per pass: every load of a pass is issued before its stores
  constexpr int kU = 8;
  for (int base = threadIdx.x; base < n; base += kU * (int)blockDim.x) {
    T kv[kU], vv[kU];
    size_t kd[kU], vd[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int it = min(base + u * (int)blockDim.x, n - 1);
      const int j = it / per_col, rem = it - j * per_col;
      const int g = rem / d, dd = rem - g * d;
      const int pos = kvl + j;
      const int blk = (pos >> 4) == (kvl >> 4) ? blk0 : blk1;
      const int slot = (kvl & 15) + j;
      const size_t sb = (size_t)kStageBlocks * l + (slot >> 4);
      kv[u] = skl[((sb * nkv + g) * kBlock + (slot & 15)) * d + dd];
      vv[u] = svl[((sb * nkv + g) * d + dd) * kBlock + (slot & 15)];
      kd[u] = (((size_t)blk * nkv + g) * kBlock + (pos & 15)) * d + dd;
      vd[u] = (((size_t)blk * nkv + g) * d + dd) * kBlock + (pos & 15);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (base + u * (int)blockDim.x < n) {
        kp[kd[u]] = kv[u];
        vp[vd[u]] = vv[u];
      }
    }
  }
}

int launch_commit_kv(const int32_t* committed, const int32_t* kv_len, const int32_t* block_table, int max_blocks,
                     int n_blocks, void* kpool, void* vpool, int n_attn, int nkv, int d, const void* sk,
                     const void* sv, size_t stage_layer_elems, const RowInfo& ri, bool bf16, hipStream_t st) {
  dim3 grid(ri.L, n_attn), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_commit_kv<bf16_t>, grid, block, 0, st, committed, kv_len, block_table, max_blocks, n_blocks,
                       reinterpret_cast<bf16_t*>(kpool), reinterpret_cast<bf16_t*>(vpool), nkv, d,
                       reinterpret_cast<const bf16_t*>(sk), reinterpret_cast<const bf16_t*>(sv),
                       stage_layer_elems, ri);
  else
    hipLaunchKernelGGL(k_commit_kv<float>, grid, block, 0, st, committed, kv_len, block_table, max_blocks, n_blocks,
                       reinterpret_cast<float*>(kpool), reinterpret_cast<float*>(vpool), nkv, d,
                       reinterpret_cast<const float*>(sk), reinterpret_cast<const float*>(sv),
                       stage_layer_elems, ri);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_kvlen_update(const int32_t* committed, int32_t* kv_len, RowInfo ri) {
  const int l = threadIdx.x;
  if (l < ri.L) kv_len[l] += max(1, min(committed[l], (int)ri.lane_cols[l]));
}

int launch_kvlen_update(const int32_t* committed, int32_t* kv_len, const RowInfo& ri, hipStream_t st) {
  hipLaunchKernelGGL(k_kvlen_update, dim3(1), dim3(64), 0, st, committed, kv_len, ri);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_sum_partials(const float* P, int S, size_t n, float* Y) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    float t = P[i];
    for (int s = 1; s < S; ++s) t += P[(size_t)s * n + i];
    Y[i] = t;
  }
}

int launch_sum_partials(const float* P, int S, size_t n, float* Y, hipStream_t st) {
  const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
  hipLaunchKernelGGL(k_sum_partials, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, P, S, n, Y);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_copy_words(const uint32_t* src, uint32_t* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

int launch_copy_rows(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_copy_words, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
